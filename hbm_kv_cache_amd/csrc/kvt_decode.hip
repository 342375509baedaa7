// kvt_decode.hip -- S6 GQA decode attention over gathered K/V (split-K, deterministic merge).
//
// QSA-KVO qsa_sparse_attend_rows_staged: query head i reads KV head i / group; each key chunk
// yields a partial (o, m, l) and the partials are folded with the online-softmax rule
// (m' = max, alpha = e^(m - m'), beta = e^(m_c - m'), a chunk with m = -inf contributes 0).
//
// decode_partial: one wavefront per (64-key chunk, KV head).  All of the chunk's K (as MFMA B
//   operands, straight from HBM) and V (staged in LDS) loads are issued up front.  The group's
//   query heads (padded to 16 rows) times K^T run on v_mfma_f32_16x16x32_{bf16,f16}: bf16/f16
//   products are exact in fp32, accumulation is fp32.  Softmax and P*V stay in fp32 on the
//   vector ALUs: with at most 16 query rows per KV head the PV product is tiny, and keeping
//   the probabilities in fp32 avoids rounding them to 16 bits.
// decode_merge: one thread per (query head, dim) folds the chunks in index order: the global
//   max first, then every chunk rescaled by e^(m_c - max) -- the same fold, one rescale each.
#include <cmath>

#include "kvt_internal.h"

namespace {

constexpr int kHd = 128;
constexpr int kKeys = 64;   // keys per chunk (4 MFMA column tiles of 16)
constexpr int kVPitch = kHd * 2 + 4;  // bytes per staged V row (padded)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(uint16_t b, bool is_bf16)
{
    return is_bf16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

template <bool kBf16>
__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c)
{
    if constexpr (kBf16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// part layout: [kvh][n_chunks][group][kHd + 2]  (o[kHd], m, l); m, l in the log2 domain
template <bool kBf16>
__global__ __launch_bounds__(64) void decode_partial(const uint16_t *__restrict__ q, int group,
                                                     const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v, int64_t n_kv,
                                                     const int32_t *__restrict__ n_valid,
                                                     float scale_log2, float *__restrict__ part)
{
    __shared__ __align__(16) unsigned char vs[kKeys * kVPitch];
    __shared__ __align__(16) float ps[kKeys][16];   // probabilities, key-major
    const int lane = threadIdx.x;
    const int c = blockIdx.x, h = blockIdx.y, n_chunks = gridDim.x;
    const int64_t key0 = (int64_t)c * kKeys;
    const int g = lane >> 4, col = lane & 15;

    // Every load below is unconditional, from a clamped (always valid) address, so all of them
    // are in flight together; out-of-range rows are zeroed or masked afterwards.
    const int qrow = col < group ? col : group - 1;
    const uint16_t *qh = q + ((int64_t)h * group + qrow) * kHd + 8 * g;
    uint4 qa[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
        qa[ks] = *reinterpret_cast<const uint4 *>(qh + ks * 32);
    const uint16_t *kh = k + (int64_t)h * n_kv * kHd;
    uint4 kb[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
        const int64_t key = min(key0 + nt * 16 + col, n_kv - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            kb[nt][ks] = *reinterpret_cast<const uint4 *>(kh + key * kHd + ks * 32 + 8 * g);
    }
    const uint16_t *vh = v + (int64_t)h * n_kv * kHd;
    uint4 vr[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int w = lane + 64 * j, row = w >> 4, cw = w & 15;
        const int64_t key = min(key0 + row, n_kv - 1);
        vr[j] = *reinterpret_cast<const uint4 *>(vh + key * kHd + cw * 8);
    }
    int64_t nv = n_valid ? (int64_t)n_valid[h] : n_kv;
    nv = nv < n_kv ? nv : n_kv;
    if (col >= group) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            qa[ks] = make_uint4(0, 0, 0, 0);
    }

    f32x4 s[4];
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
        s[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            s[nt] = mfma16x16x32<kBf16>(qa[ks], kb[nt][ks], s[nt]);
    }
    // V rows of keys that take no part are zeroed: their probability is 0, but 0 * NaN is not
    // (rows past n_valid may hold anything, e.g. slots a gather skipped)
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int w = lane + 64 * j, row = w >> 4, cw = w & 15;
        const uint4 val = key0 + row < nv ? vr[j] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(vs + row * kVPitch + cw * 16) = val;
    }

    // lane holds S[row 4g+i][key nt*16 + col]; scale into the log2 domain, mask invalid keys
    float m[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        m[i] = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
            const bool ok = key0 + nt * 16 + col < nv;
            s[nt][i] = ok ? s[nt][i] * scale_log2 : -INFINITY;
            m[i] = fmaxf(m[i], s[nt][i]);
        }
    }
    // row max / sum across the 16 lanes of a group (xor offsets stay inside the group)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
        for (int i = 0; i < 4; i++)
            m[i] = fmaxf(m[i], __shfl_xor(m[i], off, 64));
#pragma unroll
    for (int i = 0; i < 4; i++) {
        l[i] = 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
            const float p = m[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[nt][i] - m[i]);
            ps[nt * 16 + col][4 * g + i] = p;
            l[i] += p;
        }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
        for (int i = 0; i < 4; i++)
            l[i] += __shfl_xor(l[i], off, 64);
    __syncthreads();

    // O[r][2*lane .. 2*lane+1] = sum_key p[r][key] * V[key][...]
    float o[16][2];
#pragma unroll
    for (int r = 0; r < 16; r++)
        o[r][0] = o[r][1] = 0.f;
    const int nq4 = (group + 3) >> 2;   // float4 groups of probabilities actually used
#pragma unroll 4
    for (int key = 0; key < kKeys; key++) {
        const uint32_t pair = *reinterpret_cast<const uint32_t *>(vs + key * kVPitch + lane * 4);
        const float v0 = to_f32((uint16_t)(pair & 0xffff), kBf16);
        const float v1 = to_f32((uint16_t)(pair >> 16), kBf16);
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            if (q4 < nq4) {
                const float4 p = *reinterpret_cast<const float4 *>(&ps[key][4 * q4]);
                const float pr[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    o[4 * q4 + e][0] = fmaf(pr[e], v0, o[4 * q4 + e][0]);
                    o[4 * q4 + e][1] = fmaf(pr[e], v1, o[4 * q4 + e][1]);
                }
            }
        }
    }
    float *pb = part + ((int64_t)h * n_chunks + c) * group * (kHd + 2);
#pragma unroll
    for (int r = 0; r < 16; r++) {
        if (r < group)
            *reinterpret_cast<float2 *>(pb + r * (kHd + 2) + 2 * lane) = make_float2(o[r][0], o[r][1]);
    }
    if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = 4 * g + i;
            if (r < group) {
                pb[r * (kHd + 2) + kHd] = m[i];
                pb[r * (kHd + 2) + kHd + 1] = l[i];
            }
        }
    }
}

// grid = n_qh, block = kHd.  Two passes over the chunks (global max, then the weighted sums),
// each with independent loads, in chunk order: deterministic.
__global__ __launch_bounds__(kHd) void decode_merge(const float *__restrict__ part, int group,
                                                    int n_chunks, float *__restrict__ out)
{
    const int qh = blockIdx.x, d = threadIdx.x;
    const int h = qh / group, r = qh % group;
    const float *base = part + ((int64_t)h * n_chunks * group + r) * (kHd + 2);
    const int64_t cstride = (int64_t)group * (kHd + 2);
    float M = -INFINITY;
#pragma unroll 8
    for (int c = 0; c < n_chunks; c++)
        M = fmaxf(M, base[c * cstride + kHd]);
    float acc = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll 8
        for (int c = 0; c < n_chunks; c++) {
            const float *pb = base + c * cstride;
            const float mc = pb[kHd];
            const float w = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
            acc = fmaf(pb[d], w, acc);
            l = fmaf(pb[kHd + 1], w, l);
        }
    }
    out[(int64_t)qh * kHd + d] = l > 0.f ? acc / l : 0.f;
}

}  // namespace

extern "C" size_t kvt_attn_decode_ws_bytes(int32_t n_qh, int32_t hd, int64_t n_kv)
{
    if (n_qh < 1 || hd < 1 || n_kv < 0)
        return 0;
    const int64_t chunks = (n_kv + kKeys - 1) / kKeys;
    return (size_t)n_qh * (size_t)(chunks ? chunks : 1) * (size_t)(hd + 2) * sizeof(float);
}

// S6: QSA-KVO GQA decode attention with split-K partials and an online-softmax fold.
extern "C" int kvt_attn_decode(const void *q, int32_t n_qh, int32_t kvh, int32_t hd,
                               int32_t dtype, const void *k, const void *v, int64_t n_kv,
                               const int32_t *n_valid, float scale, float *out, void *ws,
                               size_t ws_bytes, void *stream)
{
    if (hd != kHd)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_decode: hd=%d (this build: 128)", hd);
    if (n_qh < 1 || kvh < 1 || n_qh % kvh || n_qh / kvh > 16 || kvh > 65535 || n_kv < 0)
        return kvt::fail(KVT_EINVAL, "kvt_attn_decode: n_qh=%d kvh=%d n_kv=%lld", n_qh, kvh,
                         (long long)n_kv);
    if (dtype != KVT_BF16 && dtype != KVT_F16)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_decode: dtype=%d", dtype);
    if (!q || !out || (n_kv && (!k || !v)))
        return kvt::fail(KVT_EINVAL, "kvt_attn_decode: null pointer");
    if (!kvt::aligned(q, 16) || !kvt::aligned(k, 16) || !kvt::aligned(v, 16))
        return kvt::fail(KVT_EALIGN, "kvt_attn_decode: q, k, v must be 16-byte aligned");
    const size_t need = kvt_attn_decode_ws_bytes(n_qh, hd, n_kv);
    if (!ws || ws_bytes < need)
        return kvt::fail(KVT_EINVAL, "kvt_attn_decode: workspace of %zu bytes, need %zu",
                         ws_bytes, need);
    const int64_t chunks = (n_kv + kKeys - 1) / kKeys;
    if (chunks > 0x7fffffff)
        return kvt::fail(KVT_ERANGE, "kvt_attn_decode: n_kv too large");
    hipStream_t s = kvt::as_stream(stream);
    const int group = n_qh / kvh;
    float *part = static_cast<float *>(ws);
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    if (chunks > 0) {
        if (dtype == KVT_BF16)
            hipLaunchKernelGGL(decode_partial<true>, dim3((unsigned)chunks, kvh), dim3(64), 0, s,
                               static_cast<const uint16_t *>(q), group,
                               static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                               n_kv, n_valid, scale_log2, part);
        else
            hipLaunchKernelGGL(decode_partial<false>, dim3((unsigned)chunks, kvh), dim3(64), 0, s,
                               static_cast<const uint16_t *>(q), group,
                               static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                               n_kv, n_valid, scale_log2, part);
        KVT_LAUNCHED("decode_partial");
    }
    hipLaunchKernelGGL(decode_merge, dim3(n_qh), dim3(kHd), 0, s, part, group, (int)chunks, out);
    KVT_LAUNCHED("decode_merge");
    return KVT_OK;
}
