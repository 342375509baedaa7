// kvt_prefill.hip -- S8 prefill flash attention over a tiered q8_0 KV cache.
//
// llama-T: cells [0, n_head) of the cache live in HBM and the rest in host memory; when an op
// reaches the host tail, the used host rows are staged into an HBM buffer once per op and the
// op reads head + staging; the output is bit-identical to an all-device cache.  Here the kernel
// takes the head and tail pointers and picks the pointer per key row, while the tiling sits at
// fixed absolute key positions -- so the same bytes meet the same arithmetic whether the tail
// is staged, read in place from host memory, or the whole cache is in HBM.
//
// Per workgroup: one KV head (blockIdx.x % kvh, so on an 8-XCD part with kvh = 8 each XCD
// streams one head's K/V through its own L2) and 128 query rows (32 queries x 4 query heads of
// the group for G = 4), one wave per 32 rows.  Per 64-key tile:
//   * each thread loads one q8_0 block (key = lane, block = wave) of K and of V -- the loads of
//     tile t+1 are issued before tile t is computed -- and dequantises it to fp16 with a
//     magic-number conversion (int8 -> 1024 + 128 + q in fp16, subtract 1152 exactly, times
//     the block scale: one rounding, to nearest): K as rows [key][d], V transposed [d][key];
//   * S^T = K Q^T on v_mfma_f32_32x32x16_f16 (K from LDS, Q held in registers);
//   * online softmax in fp32 (log2 domain, scale folded into one multiply), probabilities
//     rounded to fp16 -- and the row sums taken over the rounded values, so each output row is
//     an exact convex combination of V rows with those weights;
//   * O^T += V^T P^T on the same MFMA.  Computing S transposed leaves every lane holding the
//     16 probabilities of one query row in the MFMA B-operand layout, so P needs no shuffle:
//     the k-slots of a PV step are the keys {16s + 4g + 0..3, 16s + 8 + 4g + 0..3} (g = lane/32)
//     and the V^T operand is read with two 8-byte LDS loads from the same key set.
// No atomics, one fixed reduction order: the result is deterministic.
#include <cmath>

#include "kvt_internal.h"

namespace {

constexpr int kHd = 128;
constexpr int kKT = 64;                        // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlk = 34;                       // q8_0 block: fp16 scale + 32 int8
constexpr int kHeadBytes = (kHd / 32) * kBlk;  // one head's slice of a row: 136 bytes
constexpr int kKPitch = kHd * 2 + 16;          // LDS bytes per dequantised K row (272)
constexpr int kVtPitch = kKT * 2 + 8;          // LDS bytes per dequantised V^T row (136)
constexpr int kLdsK = kKT * kKPitch;
constexpr int kLdsV = kHd * kVtPitch;
constexpr int kOutPitch = 33;                  // floats per row of the output transpose buffer
static_assert(kWaves * 32 * kOutPitch * 4 <= kLdsK, "output staging reuses the K tile");

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The 9 dwords that cover q8_0 block b of a head slice (36 bytes from byte 4*floor(34b/4)).
__device__ __forceinline__ void load_block(const unsigned char *row, int b, uint32_t w[9])
{
    const uint32_t *p = reinterpret_cast<const uint32_t *>(row + 4 * ((kBlk * b) >> 2));
#pragma unroll
    for (int k = 0; k < 9; k++)
        w[k] = __builtin_nontemporal_load(p + k);
}

// q8_0 block -> 32 fp16 values (16 dwords, element order).  odd: the block starts 2 bytes
// into its first dword.
__device__ __forceinline__ void dequant_block(const uint32_t w[9], bool odd, uint32_t out[16])
{
    const uint16_t sbits = odd ? (uint16_t)(w[0] >> 16) : (uint16_t)(w[0] & 0xffff);
    const _Float16 s = __builtin_bit_cast(_Float16, sbits);
    const h2 s2 = {s, s};
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const uint32_t q = odd ? w[k + 1] : __builtin_amdgcn_alignbyte(w[k + 1], w[k], 2);
        const uint32_t u = q ^ 0x80808080u;                       // q + 128, as bytes
        const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
        const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
        const h2 a = (__builtin_bit_cast(h2, lo) - bias) * s2;   // exact q, then one rounding
        const h2 c = (__builtin_bit_cast(h2, hi) - bias) * s2;
        out[2 * k] = __builtin_bit_cast(uint32_t, a);
        out[2 * k + 1] = __builtin_bit_cast(uint32_t, c);
    }
}

__global__ __launch_bounds__(kThreads) void prefill_q8_0(
    const _Float16 *__restrict__ q, int64_t n_q, int64_t q_pos0, int n_qh, int kvh, int group,
    const unsigned char *__restrict__ k_head, const unsigned char *__restrict__ v_head,
    int64_t n_head, const unsigned char *__restrict__ k_tail,
    const unsigned char *__restrict__ v_tail, int64_t n_kv, int causal, float scale_log2,
    float *__restrict__ out)
{
    __shared__ __align__(16) unsigned char lds_k[kLdsK];
    __shared__ __align__(16) unsigned char lds_v[kLdsV];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, i = lane & 31;
    const int h = blockIdx.x % kvh;
    const int64_t qt = blockIdx.x / kvh;
    const int qpw = 32 * (kWaves / group);         // queries per workgroup
    const int64_t q_base = qt * qpw;
    const int qh = h * group + wave % group;        // this wave's query head
    const int64_t t_first = q_base + 32 * (wave / group);
    const int64_t t_i = t_first + i;                // this lane's query row
    const int64_t t_ld = t_i < n_q ? t_i : n_q - 1;
    const int64_t row_bytes = (int64_t)kvh * kHeadBytes;

    // last key any query of the workgroup / of this wave may see
    auto last_key_for = [&](int64_t t_last) -> int64_t {
        if (t_last > n_q - 1)
            t_last = n_q - 1;
        int64_t lk = causal ? q_pos0 + t_last : n_kv - 1;
        return lk < n_kv - 1 ? lk : n_kv - 1;
    };
    const int64_t wg_last = last_key_for(q_base + qpw - 1);
    const int64_t wave_last = t_first < n_q ? last_key_for(t_first + 31) : -1;
    const int64_t pos_first = q_pos0 + t_first;
    const int64_t pos_i = q_pos0 + t_i;
    const int n_tiles = wg_last < 0 ? 0 : (int)((wg_last + kKT) / kKT);

    // Q^T as MFMA B operands: column i = query row, k = d = 16*kd + 8*g + 0..7
    f16x8 qb[8];
    const _Float16 *qrow = q + (t_ld * n_qh + qh) * kHd + 8 * g;
#pragma unroll
    for (int kd = 0; kd < 8; kd++)
        qb[kd] = *reinterpret_cast<const f16x8 *>(qrow + 16 * kd);

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
        o[dt] = f32x16{};
    float m = -INFINITY, l = 0.f;

    // this thread's q8_0 block in the dequantisation: key = lane of the tile, block = wave
    const int blk = wave;
    const bool odd = blk & 1;
    uint32_t rk[9], rv[9];
    auto load_tile = [&](int tile) {
        int64_t key = (int64_t)tile * kKT + lane;
        key = key < n_kv ? key : n_kv - 1;
        const bool in_head = key < n_head;
        const int64_t r = in_head ? key : key - n_head;
        const unsigned char *kr = (in_head ? k_head : k_tail) + r * row_bytes + h * kHeadBytes;
        const unsigned char *vr = (in_head ? v_head : v_tail) + r * row_bytes + h * kHeadBytes;
        load_block(kr, blk, rk);
        load_block(vr, blk, rv);
    };
    if (n_tiles > 0)
        load_tile(0);

    for (int tile = 0; tile < n_tiles; tile++) {
        // dequantise this tile into LDS: K rows [key][d], V transposed [d][key]
        {
            uint32_t dk[16], dv[16];
            dequant_block(rk, odd, dk);
            dequant_block(rv, odd, dv);
            unsigned char *kdst = lds_k + lane * kKPitch + blk * 64;
#pragma unroll
            for (int c = 0; c < 4; c++)
                *reinterpret_cast<u32x4 *>(kdst + 16 * c) =
                    u32x4{dk[4 * c], dk[4 * c + 1], dk[4 * c + 2], dk[4 * c + 3]};
            unsigned char *vdst = lds_v + (blk * 32) * kVtPitch + lane * 2;
#pragma unroll
            for (int e = 0; e < 32; e++)
                *reinterpret_cast<uint16_t *>(vdst + e * kVtPitch) =
                    (uint16_t)(dv[e >> 1] >> ((e & 1) * 16));
        }
        __syncthreads();
        if (tile + 1 < n_tiles)
            load_tile(tile + 1);

        const int64_t key0 = (int64_t)tile * kKT;
        if (key0 <= wave_last) {
            // S^T tile: rows = keys 32*st + (lane & 31), columns = this wave's 32 query rows
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int kd = 0; kd < 8; kd++) {
#pragma unroll
                for (int st = 0; st < 2; st++) {
                    const f16x8 a = *reinterpret_cast<const f16x8 *>(
                        lds_k + (32 * st + i) * kKPitch + (16 * kd + 8 * g) * 2);
                    s[st] = mfma32(a, qb[kd], s[st]);
                }
            }
            // lane holds S[query i][key0 + 32*st + 8*(r/4) + 4*g + r%4] in s[st][r]
            const bool need_mask = key0 + kKT - 1 > (causal ? pos_first : n_kv - 1) ||
                                   key0 + kKT > n_kv;
            float mt = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; st++) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    float x = s[st][r] * scale_log2;
                    if (need_mask) {
                        const int64_t key = key0 + 32 * st + 8 * (r >> 2) + 4 * g + (r & 3);
                        if (key >= n_kv || (causal && key > pos_i))
                            x = -INFINITY;
                    }
                    s[st][r] = x;
                    mt = fmaxf(mt, x);
                }
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float m_new = fmaxf(m, mt);
            const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
            uint32_t pk[2][8];   // fp16 probabilities, packed in pairs
            float psum = 0.f;
#pragma unroll
            for (int st = 0; st < 2; st++) {
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = m_new == -INFINITY ? 0.f : exp2f(s[st][r] - m_new);
                    const float p1 = m_new == -INFINITY ? 0.f : exp2f(s[st][r + 1] - m_new);
                    const h2 ph = {(_Float16)p0, (_Float16)p1};
                    psum += (float)ph[0] + (float)ph[1];
                    pk[st][r >> 1] = __builtin_bit_cast(uint32_t, ph);
                }
            }
            psum += __shfl_xor(psum, 32, 64);
            l = l * alpha + psum;
            m = m_new;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < 4; dt++)
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        o[dt][r] *= alpha;
            }
            // O^T[d][query] += V^T[d][keys] P^T[keys][query], 16 keys per step
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const int st = ks >> 1, r0 = 4 * (ks & 1);
                const f16x8 pb = __builtin_bit_cast(
                    f16x8, u32x4{pk[st][r0], pk[st][r0 + 1], pk[st][r0 + 2], pk[st][r0 + 3]});
#pragma unroll
                for (int dt = 0; dt < 4; dt++) {
                    const unsigned char *vrow = lds_v + (32 * dt + i) * kVtPitch;
                    const f16x4 lo = *reinterpret_cast<const f16x4 *>(vrow + 2 * (16 * ks + 4 * g));
                    const f16x4 hi =
                        *reinterpret_cast<const f16x4 *>(vrow + 2 * (16 * ks + 8 + 4 * g));
                    const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[dt] = mfma32(a, pb, o[dt]);
                }
            }
        }
        __syncthreads();
    }

    // normalise and write O[query][qh][d] through LDS (reusing the K tile), 32 d at a time
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    float *buf = reinterpret_cast<float *>(lds_k) + wave * 32 * kOutPitch;
#pragma unroll
    for (int dt = 0; dt < 4; dt++) {
#pragma unroll
        for (int r = 0; r < 16; r++)
            buf[i * kOutPitch + 8 * (r >> 2) + 4 * g + (r & 3)] = o[dt][r] * inv_l;
        __syncthreads();
        if (t_i < n_q) {
            float *dst = out + (t_i * n_qh + qh) * kHd + 32 * dt + 16 * g;
            const float *src = buf + i * kOutPitch + 16 * g;
#pragma unroll
            for (int c = 0; c < 4; c++)
                *reinterpret_cast<float4 *>(dst + 4 * c) =
                    make_float4(src[4 * c], src[4 * c + 1], src[4 * c + 2], src[4 * c + 3]);
        }
        __syncthreads();
    }
}

}  // namespace

// S8: llama-T tiered prefill attention (HBM head + staged or host-resident tail).
extern "C" int kvt_attn_prefill(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                                int32_t kvh, int32_t hd, const void *k_head, const void *v_head,
                                int64_t n_head, const void *k_tail, const void *v_tail,
                                int64_t n_kv, int32_t kv_format, int32_t causal, float scale,
                                float *out, void *stream)
{
    if (kv_format != KVT_Q8_0)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_prefill: kv_format=%d (this build: Q8_0)",
                         kv_format);
    if (hd != kHd)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_prefill: hd=%d (this build: 128)", hd);
    if (kvh < 1 || n_qh < 1 || n_qh % kvh)
        return kvt::fail(KVT_EINVAL, "kvt_attn_prefill: n_qh=%d kvh=%d", n_qh, kvh);
    const int group = n_qh / kvh;
    if (group != 1 && group != 2 && group != 4)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_prefill: group %d (this build: 1, 2, 4)",
                         group);
    if (n_q < 0 || q_pos0 < 0 || n_kv < 0 || n_head < 0 || n_head > n_kv)
        return kvt::fail(KVT_EINVAL, "kvt_attn_prefill: n_q=%lld q_pos0=%lld n_head=%lld n_kv=%lld",
                         (long long)n_q, (long long)q_pos0, (long long)n_head, (long long)n_kv);
    if (n_q == 0)
        return KVT_OK;
    if (!q || !out || (n_head > 0 && (!k_head || !v_head)) ||
        (n_kv > n_head && (!k_tail || !v_tail)))
        return kvt::fail(KVT_EINVAL, "kvt_attn_prefill: null pointer");
    if (!kvt::aligned(q, 16) || !kvt::aligned(out, 16) || !kvt::aligned(k_head, 4) ||
        !kvt::aligned(v_head, 4) || !kvt::aligned(k_tail, 4) || !kvt::aligned(v_tail, 4))
        return kvt::fail(KVT_EALIGN, "kvt_attn_prefill: q/out need 16-byte, K/V 4-byte alignment");
    const int qpw = 32 * (kWaves / group);
    const int64_t q_tiles = (n_q + qpw - 1) / qpw;
    if (q_tiles * kvh > 0x7fffffffll)
        return kvt::fail(KVT_ERANGE, "kvt_attn_prefill: too many query tiles");
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipLaunchKernelGGL(prefill_q8_0, dim3((unsigned)(q_tiles * kvh)), dim3(kThreads), 0,
                       kvt::as_stream(stream), static_cast<const _Float16 *>(q), n_q, q_pos0,
                       n_qh, kvh, group, static_cast<const unsigned char *>(k_head),
                       static_cast<const unsigned char *>(v_head), n_head,
                       static_cast<const unsigned char *>(k_tail),
                       static_cast<const unsigned char *>(v_tail), n_kv, causal, scale_log2, out);
    KVT_LAUNCHED("prefill_q8_0");
    return KVT_OK;
}
