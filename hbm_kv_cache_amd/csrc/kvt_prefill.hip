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
// streams one head's K/V through its own L2) and 256 query rows -- for G = 4, 64 queries x the
// 4 query heads of the group -- one wave per 32 rows.  Per 64-key tile:
//   * the tile's raw q8_0 head slices (64 keys x 136 bytes per plane, 1088 bytes apart in the
//     cache rows) are read with coalesced 8-byte loads -- consecutive lanes on consecutive words
//     of one slice, so a load instruction touches a handful of cache lines rather than one per
//     lane -- and parked in LDS (fp16 / bf16 slices of 256 bytes: 16-byte loads when the cache
//     pointers are 16-byte aligned, else 8-byte ones);
//   * every thread then owns one q8_0 block of the tile (plane K or V, key = lane, block 0..3)
//     and dequantises it to fp16 with a magic-number conversion (the int8 byte under 0x64 is
//     1024 + 128 + q in fp16; subtracting 1152 is exact; times the block scale is the one
//     rounding, to nearest): K and V as rows [key][d].  Raw and fp16 tiles
//     are double buffered: tile t+1 is dequantised while tile t is multiplied, one barrier per
//     tile, with the loads of tiles t+2 and t+3 in flight;
//   * fp16 and bf16 slices need no conversion and take another schedule: the waves run as two
//     groups in alternating phases (waves w and w + 4 share a SIMD).  Waves 0-3 move the K
//     plane of each tile and lead; waves 4-7 move the V plane and trail by one phase.  A wave's
//     MFMA phase holds the V P product of the previous tile and the S product of this one, its
//     VALU phase the softmax step and its plane's store and next load, so on every SIMD one
//     wave multiplies while the other exponentiates;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_f16 (K from LDS, Q held in registers);
//   * online softmax in fp32 in the log2 domain: p = exp2(s*c - m*c) with the scale c folded
//     into one FMA and the exponential on the bare v_exp_f32 (results below 2^-126 flush to
//     zero, which no probability sum notices); probabilities rounded to fp16 in pairs;
//   * O^T += V^T P^T on the same MFMA.  Computing S transposed leaves every lane holding the
//     16 probabilities of one query row in the MFMA B-operand layout, so P needs no shuffle:
//     the k-slots of a PV step are the keys {16s + 4g + 0..3, 16s + 8 + 4g + 0..3} (g = lane/32)
//     and the V^T operand is read from the row-major V tile with two transposing 8-byte LDS
//     reads (ds_read_b64_tr_b16) from the same key set.
// No atomics, one fixed reduction order: the result is deterministic.
#include <cmath>
#include <type_traits>

#include "kvt_internal.h"

namespace {

constexpr int kHd = 128;
constexpr int kKT = 64;                        // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlk = 34;                       // q8_0 block: fp16 scale + 32 int8
constexpr int kKPitch = kHd * 2 + 16;          // LDS bytes per dequantised K row (272)
constexpr int kLdsK = kKT * kKPitch;
// LDS bytes per dequantised V row (304 = 76 dwords).  The PV product reads V transposed, each
// 16-lane group from four rows; at 76 dwords those rows overlap in fewer banks than at 272
// bytes, while sixteen rows' 16-byte stores still fall in distinct banks.  Measured against
// 272 and 320: 3% faster for q8_0 and fp16 / bf16 caches alike.
constexpr int kVPitch = kHd * 2 + 48;
constexpr int kLdsBuf = kLdsK + kKT * kVPitch;     // one tile, K and V
// The raw (as stored) tile per cache format: one head's slice of a row is four q8_0 blocks
// (136 bytes) or 128 fp16 / bf16 values (256 bytes).
constexpr int head_bytes(int fmt) { return fmt == KVT_Q8_0 ? (kHd / 32) * kBlk : kHd * 2; }
template <int F>
struct Raw {
    static constexpr int kHeadBytes = head_bytes(F);
    static constexpr int kPlane = kKT * kHeadBytes;                  // one plane's slices of a tile
    static constexpr int kBytes = 2 * kPlane;                        // K and V
};
// The raw tile as the loads see it: WB-byte words (8; 16 for fp16 / bf16 slices, which are 256
// bytes, when the cache pointers are 16-byte aligned).
template <int F, int WB>
struct Words {
    static_assert(WB == 8 || (WB == 16 && F != KVT_Q8_0), "q8_0 slices are 8-byte aligned only");
    using Word = std::conditional_t<WB == 8, uint64_t, u32x4>;
    static constexpr int kWords = Raw<F>::kBytes / WB;               // words per tile
    static constexpr int kPerThread = (kWords + kThreads - 1) / kThreads;
};
constexpr int kOutPitch = 33;                  // floats per row of the output transpose buffer
static_assert(kWaves * 32 * kOutPitch * 4 <= 2 * kLdsBuf, "output staging reuses the tiles");

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// The same product with both operands holding bf16 bit patterns.
__device__ __forceinline__ f32x16 mfma32_bf16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// x * y rounded on its own: the empty asm hides the product from contraction into a later
// fused multiply-add.
__device__ __forceinline__ float mul_rounded(float x, float y)
{
    float r = x * y;
    asm volatile("" : "+v"(r));
    return r;
}

// fp32 pairs -> bf16 pairs rounded to nearest even (bit patterns, first value low).
__device__ __forceinline__ uint32_t bf16_pair(float a, float b)
{
    auto rne = [](float x) {
        const uint32_t u = __builtin_bit_cast(uint32_t, x);
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    };
    return rne(a) | (rne(b) << 16);
}
// A value as the sum of two bf16 values: hi = bf16(x), lo = bf16(x - hi).  For an fp16 x
// (11 significant bits) the sum is exactly x; for an fp32 x it carries 16 significant bits.
__device__ __forceinline__ void bf16_split(float a, float b, uint32_t &hi, uint32_t &lo)
{
    hi = bf16_pair(a, b);
    const float ha = __builtin_bit_cast(float, hi << 16);
    const float hb = __builtin_bit_cast(float, hi & 0xffff0000u);
    lo = bf16_pair(a - ha, b - hb);
}

// x of lanes 0-31 and of lanes 32-63, each in all 64 lanes, from one v_permlane32_swap (a VALU
// exchange; no LDS round trip): lo[L] = x[L % 32], hi[L] = x[32 + L % 32].
__device__ __forceinline__ void wave_halves(float x, float &lo, float &hi)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    // scalar copies first: a bit_cast of a vector element subscript reads element 0
    const uint32_t a = r[0], b = r[1];
    lo = __builtin_bit_cast(float, a);
    hi = __builtin_bit_cast(float, b);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: in each group of 16 lanes, lane s reads 4 values and receives value s % 4
// of the reads of lanes 4e + s / 4, e = 0..3 -- one column of four rows.
__device__ __forceinline__ f16x4 tr_read(const unsigned char *p)
{
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4 *)(p)));
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


// q8_0 rows -> fp16 rows ([row][head][d], 256 bytes a head): the values dequant_block gives
// inside prefill_attn, so the fp16 kernel over converted rows computes what the q8_0 kernel
// computes over the originals.  Each workgroup reads `rows_per_group` consecutive rows into LDS
// with coalesced 8-byte loads, then each thread converts 34-byte blocks from there.  blockIdx.y
// picks the plane: (src0, dst0) or (src1, dst1).
__global__ __launch_bounds__(256) void q8_0_to_f16_rows(const unsigned char *__restrict__ src0,
                                                        const unsigned char *__restrict__ src1,
                                                        int64_t n_rows, int kvh,
                                                        int rows_per_group,
                                                        unsigned char *__restrict__ dst0,
                                                        unsigned char *__restrict__ dst1)
{
    extern __shared__ __align__(16) unsigned char conv_lds[];
    const unsigned char *const src = blockIdx.y ? src1 : src0;
    unsigned char *const dst = blockIdx.y ? dst1 : dst0;
    const int64_t row_bytes = (int64_t)kvh * (kHd / 32) * kBlk;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_group;
    const int n = (int)(n_rows - r0 < rows_per_group ? n_rows - r0 : rows_per_group);
    const int words = (int)(n * row_bytes / 8);
    const uint64_t *s8 = reinterpret_cast<const uint64_t *>(src + r0 * row_bytes);
    for (int w = threadIdx.x; w < words; w += 256)
        reinterpret_cast<uint64_t *>(conv_lds)[w] = __builtin_nontemporal_load(s8 + w);
    __syncthreads();
    // one 16-byte output chunk per thread and step, consecutive threads on consecutive chunks
    // (coalesced stores): chunk c of a row is quarter c % 4 of block c / 4 (head c / 16), the
    // block's values 8 * (c % 4) .. + 7, dequantised as dequant_block does
    const int per_row = kvh * (kHd / 32) * 4;
    unsigned char *const d0 = dst + r0 * (int64_t)kvh * kHd * 2;
    for (int c = threadIdx.x; c < n * per_row; c += 256) {
        const int row = c / per_row, cc = c - row * per_row;
        const int br = cc >> 2, qt = cc & 3;
        const int off = (int)(row * row_bytes) + kBlk * br;
        const uint32_t *w32 = reinterpret_cast<const uint32_t *>(conv_lds + (off & ~3));
        const bool odd = (off & 2) != 0;
        const uint32_t w0 = w32[0], wa = w32[2 * qt], wb = w32[2 * qt + 1], wc = w32[2 * qt + 2];
        const uint16_t sbits = odd ? (uint16_t)(w0 >> 16) : (uint16_t)(w0 & 0xffff);
        const _Float16 sc = __builtin_bit_cast(_Float16, sbits);
        const h2 s2 = {sc, sc};
        const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const uint32_t q = odd ? (k ? wc : wb)
                                   : __builtin_amdgcn_alignbyte(k ? wc : wb, k ? wb : wa, 2);
            const uint32_t u = q ^ 0x80808080u;
            const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
            const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
            o[2 * k] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(h2, lo) - bias) * s2);
            o[2 * k + 1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(h2, hi) - bias) * s2);
        }
        *reinterpret_cast<u32x4 *>(d0 + 16 * (int64_t)c) = u32x4{o[0], o[1], o[2], o[3]};
    }
}

// Coalesced WB-byte loads of tile `tile`: for q8_0 (WB 8) word f is plane f / 1088, key
// (f % 1088) / 17, byte 8 * (f % 17) of that key's 136-byte head slice.
// k_head ... v_tail already point at this workgroup's head slice (offset h * 136 added).
template <int F, int WB>
__device__ __forceinline__ void load_raw(const unsigned char *k_head, const unsigned char *v_head,
                                         const unsigned char *k_tail, const unsigned char *v_tail,
                                         int64_t n_head, int64_t n_kv, int64_t row_bytes, int tile,
                                         typename Words<F, WB>::Word (&rq)[Words<F, WB>::kPerThread])
{
    using R = Raw<F>;
    using W = Words<F, WB>;
    // the tile's first key in each tier, as scalar bases; per word only a 32-bit row offset
    const int64_t key0 = (int64_t)tile * kKT;
    const int kmax = (int)((n_kv - 1 - key0) < kKT - 1 ? (n_kv - 1 - key0) : kKT - 1);
    const int khead = (int)((n_head - key0) < kKT ? (n_head - key0) : kKT);   // keys < khead: head
    const unsigned char *hk = k_head + key0 * row_bytes, *hv = v_head + key0 * row_bytes;
    const unsigned char *tk = k_tail + (key0 - n_head) * row_bytes;
    const unsigned char *tv = v_tail + (key0 - n_head) * row_bytes;
#pragma unroll
    for (int u = 0; u < W::kPerThread; u++) {
        const int f = threadIdx.x + u * kThreads;
        if (f < W::kWords) {
            const int plane = f >= W::kWords / 2;
            const int rem = f - plane * (W::kWords / 2);
            int kin = rem / (R::kHeadBytes / WB);
            const int w = rem - kin * (R::kHeadBytes / WB);
            kin = kin < kmax ? kin : kmax;
            const unsigned char *base = kin < khead ? (plane ? hv : hk) : (plane ? tv : tk);
            const uint32_t off = (uint32_t)kin * (uint32_t)row_bytes + (uint32_t)WB * (uint32_t)w;
            rq[u] = __builtin_nontemporal_load(reinterpret_cast<const typename W::Word *>(base + off));
        }
    }
}

// Word f goes to byte WB*f: the raw tile in LDS is [plane][key][head slice].
template <int F, int WB>
__device__ __forceinline__ void store_raw(unsigned char *rawbuf,
                                          const typename Words<F, WB>::Word (&rq)[Words<F, WB>::kPerThread])
{
    using W = Words<F, WB>;
#pragma unroll
    for (int u = 0; u < W::kPerThread; u++) {
        const int f = threadIdx.x + u * kThreads;
        if (f < W::kWords)
            *reinterpret_cast<typename W::Word *>(rawbuf + WB * f) = rq[u];
    }
}

// One plane (0: K, 1: V) of tile `tile` by the 256 threads of one wave group (gi = thread index
// in the group): the same coalesced WB-byte words as load_raw, consecutive threads on
// consecutive words of a head slice.  p_head / p_tail point at this workgroup's head slice.
// off0: the thread's word offset within a tile, (gi / words per row) * row_bytes + WB * (gi % words
// per row).  A tile wholly inside one tier and inside the cache takes a scalar base and the fixed
// per-thread offsets; only the tile that straddles the tiers or the end is addressed row by row.
template <int F, int WB>
__device__ __forceinline__ void load_plane(const unsigned char *p_head, const unsigned char *p_tail,
                                           int64_t n_head, int64_t n_kv, int64_t row_bytes, int tile,
                                           int gi, uint32_t off0,
                                           typename Words<F, WB>::Word (&rq)[Words<F, WB>::kPerThread])
{
    using R = Raw<F>;
    using W = Words<F, WB>;
    constexpr int kPerRow = R::kHeadBytes / WB;
    constexpr int kRowsPerU = 256 / kPerRow;
    static_assert(W::kWords / 2 == 256 * W::kPerThread, "a plane is 256 threads' words");
    const int64_t key0 = (int64_t)tile * kKT;
    if (key0 + kKT <= n_kv && (key0 + kKT <= n_head || key0 >= n_head)) {
        // buffer loads: the tile's base in a scalar descriptor, the row step as a scalar offset
        // and off0 as the only per-thread term (offsets stay below 64 rows, far under the
        // descriptor's 2^31-byte range)
        const unsigned char *base = key0 < n_head ? p_head + key0 * row_bytes
                                                  : p_tail + (key0 - n_head) * row_bytes;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int u = 0; u < W::kPerThread; u++) {
            const int soff = (int)(u * kRowsPerU * row_bytes);
            if constexpr (WB == 16) {
                rq[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off0, soff, 2);   // nt
            } else {
                const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off0, soff, 2);
                rq[u] = __builtin_bit_cast(uint64_t, x);
            }
        }
        return;
    }
    const int kmax = (int)((n_kv - 1 - key0) < kKT - 1 ? (n_kv - 1 - key0) : kKT - 1);
    const int khead = (int)((n_head - key0) < kKT ? (n_head - key0) : kKT);
    const unsigned char *hp = p_head + key0 * row_bytes, *tp = p_tail + (key0 - n_head) * row_bytes;
#pragma unroll
    for (int u = 0; u < W::kPerThread; u++) {
        const int f = gi + 256 * u;
        int kin = f / kPerRow;
        const int w = f - kin * kPerRow;
        kin = kin < kmax ? kin : kmax;
        const uint32_t off = (uint32_t)kin * (uint32_t)row_bytes + (uint32_t)WB * (uint32_t)w;
        rq[u] = __builtin_nontemporal_load(
            reinterpret_cast<const typename W::Word *>((kin < khead ? hp : tp) + off));
    }
}

// The words of load_plane into their rows of the 16-bit tile in `buf`.
template <int F, int WB>
__device__ __forceinline__ void store_plane(unsigned char *buf, int plane, int gi,
                                            const typename Words<F, WB>::Word (&rq)[Words<F, WB>::kPerThread])
{
    using W = Words<F, WB>;
    constexpr int kPerRow = Raw<F>::kHeadBytes / WB;
    unsigned char *const base = buf + (plane ? kLdsK : 0);
    const int pitch = plane ? kVPitch : kKPitch;
#pragma unroll
    for (int u = 0; u < W::kPerThread; u++) {
        const int f = gi + 256 * u;
        const int key = f / kPerRow, w = f - key * kPerRow;
        *reinterpret_cast<typename W::Word *>(base + key * pitch + WB * w) = rq[u];
    }
}

// Thread (plane = wave / 4, block = wave % 4, key = lane) turns its 32 values of the raw q8_0
// tile into the fp16 tile used by the MFMA: the block's dequantisation, K and V both as rows
// [key][d].  (fp16 and bf16 tiles are stored from the load registers as they are.)
template <int F>
__device__ __forceinline__ void dequant_tile(const unsigned char *rawbuf, unsigned char *buf,
                                             int wave, int lane)
{
    static_assert(F == KVT_Q8_0, "only q8_0 tiles go through a raw buffer");
    using R = Raw<F>;
    const bool is_v = wave >= 4;
    const int blk = wave & 3;
    uint32_t d[16];
    const uint32_t *src = reinterpret_cast<const uint32_t *>(
        rawbuf + (is_v ? R::kPlane : 0) + lane * R::kHeadBytes + 4 * ((kBlk * blk) >> 2));
    uint32_t w[9];
#pragma unroll
    for (int k = 0; k < 9; k++)
        w[k] = src[k];
    dequant_block(w, blk & 1, d);
    unsigned char *dst = buf + (is_v ? kLdsK + lane * kVPitch : lane * kKPitch) + blk * 64;
#pragma unroll
    for (int c = 0; c < 4; c++)
        *reinterpret_cast<u32x4 *>(dst + 16 * c) =
            u32x4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]};
}

template <int F, int WB>
__global__ __launch_bounds__(kThreads) void prefill_attn(
    const _Float16 *__restrict__ q, int64_t n_q, int64_t q_pos0, int n_qh, int kvh, int group,
    const unsigned char *__restrict__ k_head, const unsigned char *__restrict__ v_head,
    int64_t n_head, const unsigned char *__restrict__ k_tail,
    const unsigned char *__restrict__ v_tail, int64_t n_kv, int causal, float scale_log2,
    int tile_begin, int tile_cap, int n_split, int tiles_per_split, float *__restrict__ state,
    int first, int last, float *__restrict__ out)
{
    using R = Raw<F>;
    // q8_0 tiles go through raw (as stored) buffers and a dequantisation; fp16 and bf16 tiles
    // are stored from the load registers straight into the 16-bit tiles
    constexpr bool kDirect = F != KVT_Q8_0;
    __shared__ __align__(16) unsigned char lds[2 * kLdsBuf + (kDirect ? 0 : 2 * R::kBytes)];
    unsigned char *const lds_raw = lds + 2 * kLdsBuf;   // two raw tiles (q8_0)

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, i = lane & 31;
    // the lane's share of a transposed V read: row offset and column within a 32-column block
    const int tr_r = (lane & 15) >> 2, tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // split-K: gridDim.x = n_split x (query tiles x kvh); split x owns key tiles
    // [x * tiles_per_split, (x + 1) * tiles_per_split) and hands its state on.  A pass over
    // tiles [tile_begin, tile_cap) takes the part of each split's tiles inside it; the split's
    // state starts in the pass that holds its first tile, and a split with no tile in the pass
    // leaves its state alone.
    const int n_wg = gridDim.x / n_split;
    const int split = blockIdx.x / n_wg;
    const int wg = blockIdx.x - split * n_wg;
    const int h = wg % kvh;
    const int64_t qt = wg / kvh;
    int tb = tile_begin, tc = tile_cap;
    if (n_split > 1) {
        const int s0 = split * tiles_per_split;
        tb = s0 > tile_begin ? s0 : tile_begin;
        tc = s0 + tiles_per_split < tile_cap ? s0 + tiles_per_split : tile_cap;
        if (tb >= tc)
            return;
        first = tb == s0;
    }
    const int qpw = 32 * (kWaves / group);         // queries per workgroup
    const int64_t q_base = qt * qpw;
    const int qh = h * group + wave % group;        // this wave's query head
    const int64_t t_first = q_base + 32 * (wave / group);
    const int64_t t_i = t_first + i;                // this lane's query row
    const int64_t t_ld = t_i < n_q ? t_i : n_q - 1;
    const int64_t row_bytes = (int64_t)kvh * R::kHeadBytes;

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
    const int n_tiles_all = wg_last < 0 ? 0 : (int)((wg_last + kKT) / kKT);
    // this call's tiles: [tb, n_tiles) (a key range of a resumable pass or a split)
    const int n_tiles = n_tiles_all < tc ? n_tiles_all : tc;

    // Q^T as MFMA B operands: column i = query row, k = d = 16*kd + 8*g + 0..7
    // bf16 caches: the fp16 query as two bf16 halves (qb high parts, qlo low parts), exactly
    constexpr bool kBf = F == KVT_BF16;
    f16x8 qb[8];
    f16x8 qlo[kBf ? 8 : 1];
    const _Float16 *qrow = q + (t_ld * n_qh + qh) * kHd + 8 * g;
#pragma unroll
    for (int kd = 0; kd < 8; kd++)
        qb[kd] = *reinterpret_cast<const f16x8 *>(qrow + 16 * kd);
    if constexpr (kBf) {
#pragma unroll
        for (int kd = 0; kd < 8; kd++) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; e++)
                bf16_split((float)qb[kd][2 * e], (float)qb[kd][2 * e + 1], hi[e], lo[e]);
            qb[kd] = __builtin_bit_cast(f16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
            qlo[kd] = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
        }
    }

    f32x16 o[4];
    float m = -INFINITY, l = 0.f;   // running max (raw logits) and sum
    // resumable passes keep (o, m, l) per lane: [workgroup][wave][66][lane], exact fp32
    float *st = state ? state + ((int64_t)blockIdx.x * kWaves + wave) * 66 * 64 + lane : nullptr;
    if (first) {
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
            o[dt] = f32x16{};
    } else {
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                o[dt][r] = st[(16 * dt + r) * 64];
        m = st[64 * 64];
        l = st[65 * 64];
    }
    // Q (and a resumed state) are in registers before any tile is loaded.  Were their loads
    // still pending at the loop, the waits before the first uses of Q and O would be placed in
    // the loop body, and on every later tile they would also wait for the prefetch loads issued
    // at the end of the tile before.
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __builtin_amdgcn_sched_barrier(0);

    // the four cache bases, moved to this workgroup's head slice
    const unsigned char *kh = k_head + h * R::kHeadBytes, *vh = v_head + h * R::kHeadBytes;
    const unsigned char *kt = k_tail + h * R::kHeadBytes, *vt = v_tail + h * R::kHeadBytes;
    typename Words<F, WB>::Word rq[Words<F, WB>::kPerThread];

    // The tile arithmetic, in three steps per tile: S = the tile's logits (MFMA), the online
    // softmax step (VALU), and O += V P (MFMA).  s carries a tile's logits from the first step to
    // the second, pk / pl its probabilities from the second to the third.
    f32x16 s[2];
    uint32_t pk[2][8];
    uint32_t pl[2][kBf ? 8 : 1];
    // S^T tile: rows = keys 32*st + (lane & 31), columns = this wave's 32 query rows
    auto s_product = [&](const unsigned char *lk) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int kd = 0; kd < 8; kd++) {
#pragma unroll
            for (int st = 0; st < 2; st++) {
                const f16x8 a = *reinterpret_cast<const f16x8 *>(
                    lk + (32 * st + i) * kKPitch + (16 * kd + 8 * g) * 2);
                if constexpr (kBf) {
                    s[st] = mfma32_bf16(a, qb[kd], s[st]);
                    s[st] = mfma32_bf16(a, qlo[kd], s[st]);
                } else {
                    s[st] = mfma32(a, qb[kd], s[st]);
                }
            }
        }
    };
    // lane holds S[query i][key0 + 32*st + 8*(r/4) + 4*g + r%4] in s[st][r]
    auto softmax_step = [&](int64_t key0) {
        const bool need_mask = key0 + kKT - 1 > (causal ? pos_first : n_kv - 1) ||
                               key0 + kKT > n_kv;
        if (need_mask) {
            // last visible key of this lane's query, relative to the tile, in [-1, 64]
            int64_t lim = (causal && pos_i < n_kv - 1 ? pos_i : n_kv - 1) - key0;
            lim = lim < -1 ? -1 : (lim > kKT ? kKT : lim);
            // the lane's part of the key index (4g) moved to the limit, so each comparison is
            // against an inline constant rather than a per-element index held in a register
            const int rel = (int)lim - 4 * g;
#pragma unroll
            for (int st = 0; st < 2; st++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (32 * st + 8 * (r >> 2) + (r & 3) > rel)
                        s[st][r] = -INFINITY;
        }
        float mt = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; st++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                mt = fmaxf(mt, s[st][r]);
        {
            float lo, hi;
            wave_halves(mt, lo, hi);
            mt = fmaxf(lo, hi);
        }
        const float m_new = fmaxf(m, mt);
        // every logit is scaled by c > 0, so the max commutes with the scaling.  The
        // probabilities are exp2(s*c - mc) with mc = round(m*c), one rounding (an FMA): they
        // are relative to the rounded reference, so the state carried from earlier tiles
        // is rebased by exp2(round(m_old*c) - round(m_new*c)) -- exactly 1 when the max is
        // unchanged.  Rebasing by exp2(m_old*c - round(m_new*c)) instead would be off by
        // m_old*c's rounding error: a drift over thousands of tiles for ordinary logits,
        // and factors of 2^4 and more for logits near 1e8.  Both products are kept whole
        // (mul_rounded: no fused multiply-add).
        // alpha without branches: for an unchanged max the exponent is exactly 0 and alpha 1
        const float mc = m_new == -INFINITY ? 0.f : mul_rounded(m_new, scale_log2);
        const float ea = __builtin_amdgcn_exp2f(mul_rounded(m, scale_log2) - mc);
        const float alpha = m == -INFINITY ? 0.f : ea;
        // probabilities packed in pairs: fp16; for bf16 caches two bf16 parts, pk + pl
        float psum = 0.f;
#pragma unroll
        for (int st = 0; st < 2; st++) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[st][r], scale_log2, -mc));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[st][r + 1], scale_log2, -mc));
                psum += p0 + p1;
                if constexpr (kBf)
                    bf16_split(p0, p1, pk[st][r >> 1], pl[st][r >> 1]);
                else
                    pk[st][r >> 1] = __builtin_bit_cast(
                        uint32_t, __builtin_convertvector(f32x2{p0, p1}, h2));
            }
        }
        {
            float lo, hi;
            wave_halves(psum, lo, hi);
            psum = lo + hi;   // this lane's sum plus lane (L ^ 32)'s, in either order
        }
        l = l * alpha + psum;
        m = m_new;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < 4; dt++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    o[dt][r] *= alpha;
        }
    };
    // O^T[d][query] += V^T[d][keys] P^T[keys][query], 16 keys per step
    auto pv_product = [&](const unsigned char *lv) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const int st = ks >> 1, r0 = 4 * (ks & 1);
            const f16x8 pb = __builtin_bit_cast(
                f16x8, u32x4{pk[st][r0], pk[st][r0 + 1], pk[st][r0 + 2], pk[st][r0 + 3]});
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                // lane L receives V[16ks + 4g + e][32dt + L % 32], e = 0..3 (and keys + 8):
                // in its 16-lane group it reads 4 values of row 16ks + 4g + tr_r at column
                // 32dt + tr_c, and the read transposes them
                const unsigned char *vp = lv + (16 * ks + 4 * g + tr_r) * kVPitch +
                                          2 * (32 * dt + tr_c);
                const f16x4 lo = tr_read(vp), hi = tr_read(vp + 8 * kVPitch);
                const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                if constexpr (kBf) {
                    const f16x8 pbl = __builtin_bit_cast(
                        f16x8, u32x4{pl[st][r0], pl[st][r0 + 1], pl[st][r0 + 2], pl[st][r0 + 3]});
                    o[dt] = mfma32_bf16(a, pb, o[dt]);
                    o[dt] = mfma32_bf16(a, pbl, o[dt]);
                } else {
                    o[dt] = mfma32(a, pb, o[dt]);
                }
            }
        }
    };

    const int b0 = tb;
    if constexpr (kDirect) {
        // fp16 and bf16 tiles: two wave groups in alternating phases.  Waves w and w + 4 share a
        // SIMD; waves 0-3 (group 0) move the K plane of every tile and lead, waves 4-7 (group 1)
        // move the V plane and trail by one phase.  Each tile takes two phases per wave, each
        // ended by a workgroup barrier:
        //   MFMA phase of tile t: O += V P for tile t - 1, then S for tile t;
        //   VALU phase of tile t: the softmax step of tile t; the group's plane of tile t + 1
        //                         stored from the registers into buffer (t + 1) & 1; the loads
        //                         of its plane of tile t + 2 issued.
        // So on every SIMD one wave multiplies while the other runs its softmax step.  Barrier
        // by barrier: group 0 runs tile t's MFMA phase in interval 2t and its VALU phase in
        // 2t + 1, group 1 one interval later.  K(t) is read in intervals 2t and 2t + 1 and
        // K(t + 2) stored into its buffer in 2t + 3; V(t) is stored in 2t and read in 2t + 2
        // and 2t + 3, V(t + 2) stored in 2t + 4.  Double buffering suffices for both planes.
        // the group is uniform in a wave: readfirstlane makes its branches scalar, so a wave of
        // the other group jumps over the extra barriers rather than meeting them with no lanes on
        const int grp = __builtin_amdgcn_readfirstlane(wave >> 2), gi = threadIdx.x & 255;
        const unsigned char *ph = grp ? vh : kh, *pt = grp ? vt : kt;
        constexpr int kPerRow = R::kHeadBytes / WB;
        const uint32_t off0 = (uint32_t)(gi / kPerRow) * (uint32_t)row_bytes + (uint32_t)(WB * (gi % kPerRow));
        if (n_tiles > b0) {
            load_plane<F, WB>(ph, pt, n_head, n_kv, row_bytes, b0, gi, off0, rq);
            if (grp == 0) {
                store_plane<F, WB>(lds + (b0 & 1) * kLdsBuf, 0, gi, rq);
                if (n_tiles > b0 + 1)
                    load_plane<F, WB>(ph, pt, n_head, n_kv, row_bytes, b0 + 1, gi, off0, rq);
            }
        }
        __syncthreads();
        if (grp == 1) {   // the trailing group's VALU phase of tile b0 - 1: only the moves
            if (n_tiles > b0) {
                store_plane<F, WB>(lds + (b0 & 1) * kLdsBuf, 1, gi, rq);
                if (n_tiles > b0 + 1)
                    load_plane<F, WB>(ph, pt, n_head, n_kv, row_bytes, b0 + 1, gi, off0, rq);
            }
            __syncthreads();
        }
        for (int tile = b0; tile < n_tiles; tile++) {
            const int64_t key0 = (int64_t)tile * kKT;
            if (tile > b0 && key0 - kKT <= wave_last)
                pv_product(lds + ((tile - 1) & 1) * kLdsBuf + kLdsK);
            if (key0 <= wave_last)
                s_product(lds + (tile & 1) * kLdsBuf);
            __syncthreads();
            if (key0 <= wave_last)
                softmax_step(key0);
            if (tile + 1 < n_tiles)
                store_plane<F, WB>(lds + ((tile + 1) & 1) * kLdsBuf, grp, gi, rq);
            if (tile + 2 < n_tiles)
                load_plane<F, WB>(ph, pt, n_head, n_kv, row_bytes, tile + 2, gi, off0, rq);
            __syncthreads();
        }
        if (n_tiles > b0 && (int64_t)(n_tiles - 1) * kKT <= wave_last)
            pv_product(lds + ((n_tiles - 1) & 1) * kLdsBuf + kLdsK);
        if (grp == 0)   // the leading group matches the trailing group's extra barrier
            __syncthreads();
        __syncthreads();   // every product done before the output staging reuses the tiles
    } else {
        // q8_0: raw tile b -> LDS; fp16 tile b and raw tile b+1 ready; loads of b+2 in flight
        // (b = tb; buffers are indexed by tile & 1)
        if (n_tiles > b0) {
            load_raw<F, WB>(kh, vh, kt, vt, n_head, n_kv, row_bytes, b0, rq);
            store_raw<F, WB>(lds_raw + (b0 & 1) * R::kBytes, rq);
            if (n_tiles > b0 + 1)
                load_raw<F, WB>(kh, vh, kt, vt, n_head, n_kv, row_bytes, b0 + 1, rq);
        }
        __syncthreads();
        if (n_tiles > b0) {
            dequant_tile<F>(lds_raw + (b0 & 1) * R::kBytes, lds + (b0 & 1) * kLdsBuf, wave, lane);
            if (n_tiles > b0 + 1)
                store_raw<F, WB>(lds_raw + ((b0 + 1) & 1) * R::kBytes, rq);
            if (n_tiles > b0 + 2)
                load_raw<F, WB>(kh, vh, kt, vt, n_head, n_kv, row_bytes, b0 + 2, rq);
        }
        __syncthreads();

        // per tile: multiply fp16 buffer (tile & 1); dequantise raw tile+1 into the other fp16
        // buffer; move the registers of tile+2 into the raw buffer tile+1 just left; one
        // barrier; then issue the loads of tile+3
        const bool dequant_first = wave >= 4;
        for (int tile = b0; tile < n_tiles; tile++) {
            const unsigned char *lk = lds + (tile & 1) * kLdsBuf;
            const int64_t key0 = (int64_t)tile * kKT;
            // Waves w and w + 4 share a SIMD.  The upper four dequantise the next tile before
            // they multiply this one and the lower four after, so on every SIMD one wave's MFMA
            // work meets the other's VALU work.
            if (dequant_first && tile + 1 < n_tiles)
                dequant_tile<F>(lds_raw + ((tile + 1) & 1) * R::kBytes,
                                lds + ((tile + 1) & 1) * kLdsBuf, wave, lane);
            if (key0 <= wave_last) {
                s_product(lk);
                softmax_step(key0);
                pv_product(lk + kLdsK);
            }
            if (!dequant_first && tile + 1 < n_tiles)
                dequant_tile<F>(lds_raw + ((tile + 1) & 1) * R::kBytes,
                                lds + ((tile + 1) & 1) * kLdsBuf, wave, lane);
            if (tile + 2 < n_tiles)   // last, so the loads of tile + 2 have had the whole tile
                store_raw<F, WB>(lds_raw + (tile & 1) * R::kBytes, rq);
            __syncthreads();
            if (tile + 3 < n_tiles)
                load_raw<F, WB>(kh, vh, kt, vt, n_head, n_kv, row_bytes, tile + 3, rq);
        }
    }

    if (!last) {   // hand the state to the next pass
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                st[(16 * dt + r) * 64] = o[dt][r];
        st[64 * 64] = m;
        st[65 * 64] = l;
        return;
    }
    // normalise and write O[query][qh][d] through LDS (reusing the tiles), 32 d at a time
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    float *buf = reinterpret_cast<float *>(lds) + wave * 32 * kOutPitch;
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

// Split-K merge: one thread per lane of each (workgroup, wave) of the split launch.  The
// splits' (o, m, l) -- o and l relative to 2^round(m*c) -- fold in split order: M = max m_s,
// then o = sum o_s w_s, l = sum l_s w_s with w_s = 2^(round(m_s*c) - round(M*c)); a split that
// saw no key (m = -inf) weighs 0.  The result, o / l, goes to out[t][qh][d] with the kernel's
// own lane mapping (query row lane % 32, dims 32*dt + 8*(r/4) + 4*(lane/32) + r%4).
__global__ __launch_bounds__(64) void prefill_split_merge(const float *__restrict__ state,
                                                          int n_split, int kvh, int group,
                                                          int64_t n_q, int n_qh,
                                                          float scale_log2,
                                                          float *__restrict__ out)
{
    const int lane = threadIdx.x, wave = blockIdx.y, wg = blockIdx.x, n_wg = gridDim.x;
    const int64_t wstride = (int64_t)kWaves * 66 * 64;   // one workgroup's state
    const float *base = state + (int64_t)wg * wstride + (int64_t)wave * 66 * 64 + lane;
    const int64_t sstride = (int64_t)n_wg * wstride;      // one split's state
    float M = -INFINITY;
    for (int x = 0; x < n_split; x++)
        M = fmaxf(M, base[x * sstride + 64 * 64]);
    float acc[64], L = 0.f;
#pragma unroll
    for (int j = 0; j < 64; j++)
        acc[j] = 0.f;
    for (int x = 0; x < n_split; x++) {
        const float *b = base + x * sstride;
        const float mx = b[64 * 64];
        // o_s and l_s are relative to round(m_s * c) (see prefill_attn): rebase by the same
        const float w = mx == -INFINITY ? 0.f
                                        : __builtin_amdgcn_exp2f(mul_rounded(mx, scale_log2) -
                                                                 mul_rounded(M, scale_log2));
        L = fmaf(b[65 * 64], w, L);
#pragma unroll
        for (int j = 0; j < 64; j++)
            acc[j] = fmaf(b[j * 64], w, acc[j]);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int h = wg % kvh;
    const int64_t qt = wg / kvh;
    const int qpw = 32 * (kWaves / group);
    const int qh = h * group + wave % group;
    const int64_t t = qt * qpw + 32 * (wave / group) + (lane & 31);
    if (t >= n_q)
        return;
    float *dst = out + (t * n_qh + qh) * kHd + 4 * (lane >> 5);
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            dst[32 * dt + 8 * (r >> 2) + (r & 3)] = acc[16 * dt + r] * inv;
}

// splits for a launch of n_wg workgroups over n_tiles key tiles: enough to put about one
// workgroup on every CU, each split at least 8 tiles
void split_plan(int64_t n_wg, int64_t n_tiles, int &n_split, int &tiles_per_split)
{
    constexpr int64_t kTargetWg = 256;
    int64_t want = (kTargetWg + n_wg - 1) / n_wg;
    const int64_t most = n_tiles / 8;
    want = want < most ? want : most;
    want = want < 1 ? 1 : want;
    tiles_per_split = (int)((n_tiles + want - 1) / want);
    n_split = (int)((n_tiles + tiles_per_split - 1) / tiles_per_split);
}

// Argument checks shared by the prefill entry points; fills group and q_tiles.
int check_prefill(const char *fn, const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                  int32_t kvh, int32_t hd, const void *k_head, const void *v_head, int64_t n_head,
                  const void *k_tail, const void *v_tail, int64_t n_kv, int32_t kv_format,
                  float scale, const float *out, int &group, int64_t &q_tiles)
{
    if (kv_format != KVT_Q8_0 && kv_format != KVT_F16 && kv_format != KVT_BF16)
        return kvt::fail(KVT_EUNSUPPORTED, "%s: kv_format=%d (supported: Q8_0, F16, BF16)", fn,
                         kv_format);
    if (hd != kHd)
        return kvt::fail(KVT_EUNSUPPORTED, "%s: hd=%d (supported: 128)", fn, hd);
    if (kvh < 1 || n_qh < 1 || n_qh % kvh)
        return kvt::fail(KVT_EINVAL, "%s: n_qh=%d kvh=%d", fn, n_qh, kvh);
    group = n_qh / kvh;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return kvt::fail(KVT_EUNSUPPORTED, "%s: group %d (supported: 1, 2, 4, 8)", fn, group);
    if (!(scale > 0.f))
        return kvt::fail(KVT_EINVAL, "%s: scale must be positive", fn);
    if (n_q < 0 || q_pos0 < 0 || n_kv < 0 || n_head < 0 || n_head > n_kv)
        return kvt::fail(KVT_EINVAL, "%s: n_q=%lld q_pos0=%lld n_head=%lld n_kv=%lld", fn,
                         (long long)n_q, (long long)q_pos0, (long long)n_head, (long long)n_kv);
    if (n_q > 0 && (!q || !out || (n_head > 0 && (!k_head || !v_head)) ||
                    (n_kv > n_head && (!k_tail || !v_tail))))
        return kvt::fail(KVT_EINVAL, "%s: null pointer", fn);
    if (!kvt::aligned(q, 16) || !kvt::aligned(out, 16) || !kvt::aligned(k_head, 8) ||
        !kvt::aligned(v_head, 8) || !kvt::aligned(k_tail, 8) || !kvt::aligned(v_tail, 8))
        return kvt::fail(KVT_EALIGN, "%s: q/out need 16-byte, K/V 8-byte alignment", fn);
    const int qpw = 32 * (kWaves / group);
    q_tiles = (n_q + qpw - 1) / qpw;
    if (q_tiles * kvh > 0x7fffffffll || n_kv / kKT > 0x7ffffff0ll)
        return kvt::fail(KVT_ERANGE, "%s: too many query or key tiles", fn);
    return KVT_OK;
}

size_t state_bytes(int64_t q_tiles, int32_t kvh)
{
    return (size_t)q_tiles * (size_t)kvh * kWaves * 66 * 64 * sizeof(float);
}

void launch_prefill(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh, int32_t kvh,
                    int group, int64_t q_tiles, const void *k_head, const void *v_head,
                    int64_t n_head, const void *k_tail, const void *v_tail, int64_t n_kv,
                    int causal, float scale, int64_t key_begin, int64_t key_end, float *state,
                    int first, int last, float *out, int32_t kv_format, hipStream_t s,
                    int n_split = 1, int tiles_per_split = 0)
{
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    const int tile_begin = (int)(key_begin / kKT);
    const int tile_cap = (int)((key_end + kKT - 1) / kKT);
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)(q_tiles * kvh * n_split)), dim3(kThreads), 0, s,
                           static_cast<const _Float16 *>(q), n_q, q_pos0, n_qh, kvh, group,
                           static_cast<const unsigned char *>(k_head),
                           static_cast<const unsigned char *>(v_head), n_head,
                           static_cast<const unsigned char *>(k_tail),
                           static_cast<const unsigned char *>(v_tail), n_kv, causal, scale_log2,
                           tile_begin, tile_cap, n_split, tiles_per_split, state, first, last,
                           out);
    };
    // fp16 / bf16 slices are 256 bytes: 16-byte loads when every cache pointer allows them
    const bool w16 = kvt::aligned(k_head, 16) && kvt::aligned(v_head, 16) &&
                     kvt::aligned(k_tail, 16) && kvt::aligned(v_tail, 16);
    if (kv_format == KVT_Q8_0)
        launch(prefill_attn<KVT_Q8_0, 8>);
    else if (kv_format == KVT_F16)
        w16 ? launch(prefill_attn<KVT_F16, 16>) : launch(prefill_attn<KVT_F16, 8>);
    else
        w16 ? launch(prefill_attn<KVT_BF16, 16>) : launch(prefill_attn<KVT_BF16, 8>);
}

// A first bucket copied ahead by one pipelined call for the next call on the same thread: the
// host rows [0, rows) of the planes at k_host / v_host, now at the start of arena_k / arena_v.
struct Prefetched {
    int device = -1;
    uintptr_t k_host = 0, v_host = 0, arena_k = 0, arena_v = 0;
    int64_t row_bytes = 0, rows = 0;
};

// Events of the pipelined entry points, created once per thread and device and then reused:
// [0] start, [1 + slot] slot filled, [3 + slot] slot free, [5] prefetch done.
struct PipeEvents {
    int device = -1;
    hipEvent_t e[6] = {};
    Prefetched pre;   // valid for the next pipelined call on this thread only
};
thread_local PipeEvents t_pipe;

int pipe_events(hipEvent_t *&ev)
{
    int dev = 0;
    KVT_HIP(hipGetDevice(&dev));
    if (t_pipe.device != dev) {
        for (hipEvent_t &x : t_pipe.e) {
            if (x)
                (void)hipEventDestroy(x);
            x = nullptr;
        }
        t_pipe.device = -1;
        t_pipe.pre = Prefetched{};
        for (hipEvent_t &x : t_pipe.e)
            KVT_HIP(hipEventCreateWithFlags(&x, hipEventDisableTiming));
        t_pipe.device = dev;
    }
    ev = t_pipe.e;
    return KVT_OK;
}

}  // namespace

// S8: llama-T tiered prefill attention (HBM head + staged or host-resident tail).
extern "C" int kvt_attn_prefill(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                                int32_t kvh, int32_t hd, const void *k_head, const void *v_head,
                                int64_t n_head, const void *k_tail, const void *v_tail,
                                int64_t n_kv, int32_t kv_format, int32_t causal, float scale,
                                float *out, void *stream)
{
    int group = 0;
    int64_t q_tiles = 0;
    const int rc = check_prefill("kvt_attn_prefill", q, n_q, q_pos0, n_qh, kvh, hd, k_head,
                                 v_head, n_head, k_tail, v_tail, n_kv, kv_format, scale, out,
                                 group, q_tiles);
    if (rc != KVT_OK || n_q == 0)
        return rc;
    launch_prefill(q, n_q, q_pos0, n_qh, kvh, group, q_tiles, k_head, v_head, n_head, k_tail,
                   v_tail, n_kv, causal, scale, 0, n_kv, nullptr, 1, 1, out, kv_format,
                   kvt::as_stream(stream));
    KVT_LAUNCHED("prefill_attn");
    return KVT_OK;
}

// S8 for short chunks (down to single-token decode over a tiered cache): the same attention
// split over the key range when query tiles x KV heads would leave most CUs idle.
extern "C" size_t kvt_attn_prefill_splitk_ws_bytes(int64_t n_q, int32_t n_qh, int32_t kvh,
                                                   int64_t n_kv)
{
    if (n_q < 1 || n_kv < 1 || kvh < 1 || n_qh < kvh || n_qh % kvh)
        return 0;
    const int group = n_qh / kvh;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return 0;
    const int qpw = 32 * (kWaves / group);
    const int64_t q_tiles = (n_q + qpw - 1) / qpw;
    int n_split = 1, tps = 0;
    split_plan(q_tiles * kvh, (n_kv + kKT - 1) / kKT, n_split, tps);
    return n_split > 1 ? (size_t)n_split * state_bytes(q_tiles, kvh) : 0;
}

extern "C" int kvt_attn_prefill_splitk(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                                       int32_t kvh, int32_t hd, const void *k_head,
                                       const void *v_head, int64_t n_head, const void *k_tail,
                                       const void *v_tail, int64_t n_kv, int32_t kv_format,
                                       int32_t causal, float scale, void *ws, size_t ws_bytes,
                                       float *out, void *stream)
{
    int group = 0;
    int64_t q_tiles = 0;
    const int rc = check_prefill("kvt_attn_prefill_splitk", q, n_q, q_pos0, n_qh, kvh, hd,
                                 k_head, v_head, n_head, k_tail, v_tail, n_kv, kv_format, scale,
                                 out, group, q_tiles);
    if (rc != KVT_OK || n_q == 0)
        return rc;
    hipStream_t s = kvt::as_stream(stream);
    int n_split = 1, tps = 0;
    split_plan(q_tiles * kvh, (n_kv + kKT - 1) / kKT, n_split, tps);
    if (n_split == 1) {   // enough workgroups already: the single pass
        launch_prefill(q, n_q, q_pos0, n_qh, kvh, group, q_tiles, k_head, v_head, n_head, k_tail,
                       v_tail, n_kv, causal, scale, 0, n_kv, nullptr, 1, 1, out, kv_format, s);
        KVT_LAUNCHED("prefill_attn");
        return KVT_OK;
    }
    const size_t need = (size_t)n_split * state_bytes(q_tiles, kvh);
    if (!ws || ws_bytes < need || !kvt::aligned(ws, 4))
        return kvt::fail(KVT_EINVAL, "kvt_attn_prefill_splitk: workspace of %zu bytes, need %zu",
                         ws_bytes, need);
    if (q_tiles * kvh * n_split > 0x7fffffffll)
        return kvt::fail(KVT_ERANGE, "kvt_attn_prefill_splitk: too many workgroups");
    float *state = static_cast<float *>(ws);
    launch_prefill(q, n_q, q_pos0, n_qh, kvh, group, q_tiles, k_head, v_head, n_head, k_tail,
                   v_tail, n_kv, causal, scale, 0, n_kv, state, 1, 0, out, kv_format, s, n_split,
                   tps);
    KVT_LAUNCHED("prefill_attn");
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipLaunchKernelGGL(prefill_split_merge, dim3((unsigned)(q_tiles * kvh), kWaves), dim3(64), 0,
                       s, state, n_split, (int)kvh, group, n_q, (int)n_qh, scale_log2, out);
    KVT_LAUNCHED("prefill_split_merge");
    return KVT_OK;
}

extern "C" size_t kvt_attn_prefill_state_bytes(int64_t n_q, int32_t n_qh, int32_t kvh)
{
    if (n_q < 0 || kvh < 1 || n_qh < kvh || n_qh % kvh)
        return 0;
    const int group = n_qh / kvh;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return 0;
    const int qpw = 32 * (kWaves / group);
    return state_bytes((n_q + qpw - 1) / qpw, kvh);
}

// S8 as resumable passes over key ranges (the online-softmax fold over buckets of the pages'
// bounded staging arena).
extern "C" int kvt_attn_prefill_range(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                                      int32_t kvh, int32_t hd, const void *k_head,
                                      const void *v_head, int64_t n_head, const void *k_tail,
                                      const void *v_tail, int64_t n_kv, int32_t kv_format,
                                      int32_t causal, float scale, int64_t key_begin,
                                      int64_t key_end, void *state, size_t state_bytes_,
                                      float *out, void *stream)
{
    int group = 0;
    int64_t q_tiles = 0;
    const int rc = check_prefill("kvt_attn_prefill_range", q, n_q, q_pos0, n_qh, kvh, hd,
                                 k_head, v_head, n_head, k_tail, v_tail, n_kv, kv_format, scale,
                                 out, group, q_tiles);
    if (rc != KVT_OK)
        return rc;
    if (key_begin < 0 || key_end < key_begin || key_end > n_kv || key_begin % kKT ||
        (key_end % kKT && key_end != n_kv))
        return kvt::fail(KVT_EINVAL,
                         "kvt_attn_prefill_range: keys [%lld, %lld) of %lld: the bounds must be "
                         "multiples of 64 (the end may be n_kv)",
                         (long long)key_begin, (long long)key_end, (long long)n_kv);
    const int first = key_begin == 0, last = key_end == n_kv;
    if (!(first && last)) {
        if (!state || state_bytes_ < state_bytes(q_tiles, kvh) || !kvt::aligned(state, 4))
            return kvt::fail(KVT_EINVAL, "kvt_attn_prefill_range: state of %zu bytes, need %zu",
                             state_bytes_, state_bytes(q_tiles, kvh));
    }
    if (n_q == 0)
        return KVT_OK;
    launch_prefill(q, n_q, q_pos0, n_qh, kvh, group, q_tiles, k_head, v_head, n_head, k_tail,
                   v_tail, n_kv, causal, scale, key_begin, key_end, static_cast<float *>(state),
                   first, last, out, kv_format, kvt::as_stream(stream));
    KVT_LAUNCHED("prefill_attn");
    return KVT_OK;
}

namespace {

// The next call's first host rows, copied at the end of this call (rows 0: no prefetch).
struct NextBucket {
    uintptr_t k_host = 0, v_host = 0, arena_k = 0, arena_v = 0;
    int64_t rows = 0, arena_rows = 0;
};

// fp16 copies a pipelined call over a q8_0 cache converts its rows into, so that every pass
// runs the fp16 kernel (head_k null: no conversion).  head_*: n_head rows each; slot_*: the
// arena's two buckets, slot_keys rows each; rows of kvh * 256 bytes.
struct Conv {
    unsigned char *head_k = nullptr, *head_v = nullptr, *slot_k = nullptr, *slot_v = nullptr;
};

// rows [0, n) of two planes of q8_0 rows (src_k, src_v) -> fp16 rows (dst_k, dst_v), one
// launch on stream s
void convert_rows(const void *src_k, const void *src_v, int64_t n, int kvh, void *dst_k,
                  void *dst_v, hipStream_t s)
{
    if (n <= 0)
        return;
    const int64_t row_bytes = (int64_t)kvh * (kHd / 32) * kBlk;
    const int rpg = (int)std::max<int64_t>(1, std::min<int64_t>(64, 32768 / row_bytes));
    hipLaunchKernelGGL(q8_0_to_f16_rows, dim3((unsigned)((n + rpg - 1) / rpg), 2), dim3(256),
                       (size_t)(rpg * row_bytes + 16), s,
                       static_cast<const unsigned char *>(src_k),
                       static_cast<const unsigned char *>(src_v), n, kvh, rpg,
                       static_cast<unsigned char *>(dst_k), static_cast<unsigned char *>(dst_v));
}

bool ranges_overlap(uintptr_t a, uint64_t an, uintptr_t b, uint64_t bn)
{
    return an && bn && a < b + bn && b < a + an;
}

// S7+S8 overlapped (llama-T staging, with QSA-KVO's bounded arena and online-softmax fold over
// buckets, and exl3-DMA's copy of the next layer's first batch while this layer is attended).  The first
// `staged` host rows of bucket 0 are already in the arena (a previous call's prefetch).
int prefill_pipeline(const char *fn, const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                     int32_t kvh, int32_t hd, const void *k_head, const void *v_head,
                     int64_t n_head, const void *k_host, const void *v_host, int64_t n_kv,
                     int32_t kv_format, int32_t causal, float scale, void *arena_k,
                     void *arena_v, int64_t arena_rows, int64_t staged, const NextBucket &nx,
                     void *state, size_t state_bytes_, float *out, void *stream,
                     void *copy_stream, bool split_k = false, const Conv *conv = nullptr)
{
    // whatever this call does, a prefetch left by the previous one is good for it alone
    const Prefetched got = t_pipe.pre;
    t_pipe.pre = Prefetched{};
    int group = 0;
    int64_t q_tiles = 0;
    const int rc = check_prefill(fn, q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head,
                                 k_host, v_host, n_kv, kv_format, scale, out, group, q_tiles);
    if (rc != KVT_OK)
        return rc;
    if (staged < 0 || nx.rows < 0)
        return kvt::fail(KVT_EINVAL, "%s: negative row count", fn);
    hipStream_t s = kvt::as_stream(stream), cs = kvt::as_stream(copy_stream);
    const bool prefetch = nx.rows > 0;
    if (n_q == 0 && !staged && !prefetch)
        return KVT_OK;
    const bool host_rows = n_head < n_kv;
    const int64_t row_bytes = (int64_t)kvh * head_bytes(kv_format);
    const uintptr_t ak = reinterpret_cast<uintptr_t>(arena_k);
    const uintptr_t av = reinterpret_cast<uintptr_t>(arena_v);
    const uintptr_t hk = reinterpret_cast<uintptr_t>(k_host);
    const uintptr_t hv = reinterpret_cast<uintptr_t>(v_host);
    const int64_t slot_keys = arena_rows / 2 / kKT * kKT;
    const int64_t hb = n_head / kKT * kKT;   // head keys in whole tiles; the rest by bucket
    // split_k: every pass runs in kvt_attn_prefill_splitk's key splits, each split's state
    // carried from bucket to bucket, and one merge at the end (its bits, not the single pass's)
    int n_split = 1, tps = 0;
    if (split_k)
        split_plan(q_tiles * kvh, (n_kv + kKT - 1) / kKT, n_split, tps);
    if (n_split > 1 && q_tiles * kvh * n_split > 0x7fffffffll)
        return kvt::fail(KVT_ERANGE, "%s: too many workgroups", fn);
    const size_t need_state = (size_t)n_split * state_bytes(q_tiles, kvh);
    if (host_rows) {
        if (slot_keys < kKT || !arena_k || !arena_v || !kvt::aligned(arena_k, 8) ||
            !kvt::aligned(arena_v, 8))
            return kvt::fail(KVT_EINVAL,
                             "%s: arena of %lld rows (need >= 128, 8-byte aligned K and V)", fn,
                             (long long)arena_rows);
    }
    if ((host_rows || n_split > 1) && n_q > 0 &&
        (!state || state_bytes_ < need_state || !kvt::aligned(state, 4)))
        return kvt::fail(KVT_EINVAL, "%s: state of %zu bytes, need %zu", fn, state_bytes_,
                         need_state);
    if ((host_rows || prefetch) && cs == s)
        return kvt::fail(KVT_EINVAL, "%s: copy_stream must differ from stream", fn);
    if (staged) {
        // host rows of bucket 0: keys [hb, hb + slot_keys) past the head
        const int64_t b0 = host_rows ? (hb + slot_keys < n_kv ? hb + slot_keys : n_kv) - n_head
                                     : 0;
        if (got.rows != staged || got.k_host != hk || got.v_host != hv || got.arena_k != ak ||
            got.arena_v != av || got.row_bytes != row_bytes)
            return kvt::fail(KVT_EINVAL,
                             "%s: %lld rows said to be staged, but the previous pipelined call "
                             "on this thread prefetched %lld rows for other planes or arena",
                             fn, (long long)staged, (long long)got.rows);
        if (staged > b0)
            return kvt::fail(KVT_EINVAL, "%s: %lld staged rows, but the first bucket holds %lld "
                                         "host rows", fn, (long long)staged, (long long)b0);
    }
    if (prefetch) {
        const int64_t nslot = nx.arena_rows / 2 / kKT * kKT;
        if (nslot < kKT || !nx.arena_k || !nx.arena_v || !nx.k_host || !nx.v_host ||
            nx.arena_k % 8 || nx.arena_v % 8)
            return kvt::fail(KVT_EINVAL, "%s: next arena of %lld rows (need >= 128, 8-byte "
                                         "aligned K and V) and next host planes", fn,
                             (long long)nx.arena_rows);
        if (nx.rows > nslot)
            return kvt::fail(KVT_EINVAL, "%s: %lld rows to prefetch, but a bucket of the next "
                                         "arena holds %lld", fn, (long long)nx.rows,
                             (long long)nslot);
        const uint64_t nb = (uint64_t)nx.rows * (uint64_t)row_bytes;
        const uint64_t span = host_rows ? 2 * (uint64_t)slot_keys * (uint64_t)row_bytes : 0;
        if (ranges_overlap(nx.arena_k, nb, ak, span) || ranges_overlap(nx.arena_k, nb, av, span) ||
            ranges_overlap(nx.arena_v, nb, ak, span) || ranges_overlap(nx.arena_v, nb, av, span) ||
            ranges_overlap(nx.arena_k, nb, nx.arena_v, nb))
            return kvt::fail(KVT_EINVAL, "%s: the next arena overlaps this call's arena, or its "
                                         "K rows overlap its V rows", fn);
    }
    int dev = 0;
    KVT_HIP(hipGetDevice(&dev));
    if (staged && got.device != dev)
        return kvt::fail(KVT_EINVAL, "%s: the staged rows were prefetched on device %d, not %d",
                         fn, got.device, dev);
    hipEvent_t *ev = nullptr;
    if (pipe_events(ev) != KVT_OK)
        return KVT_EHIP;
    float *stf = static_cast<float *>(state);

    // the copies start after everything already on `stream` (the tail's producers, and the
    // previous calls' passes over this arena and the next one)
    if (host_rows || prefetch) {
        KVT_HIP(hipEventRecord(ev[0], s));
        KVT_HIP(hipStreamWaitEvent(cs, ev[0], 0));
    }
    const int fin = n_split > 1 ? 0 : 1;   // split passes always hand their state on
    // with a conversion, every pass reads fp16 rows: the head converted here, each bucket as
    // it lands in the arena
    const bool cv = conv && conv->head_k && kv_format == KVT_Q8_0 && n_q > 0;
    const int32_t pass_fmt = cv ? KVT_F16 : kv_format;
    const int64_t row16 = (int64_t)kvh * kHd * 2;
    const void *ph_k = cv ? conv->head_k : k_head, *ph_v = cv ? conv->head_v : v_head;
    if (cv && n_head > 0) {
        convert_rows(k_head, v_head, n_head, kvh, conv->head_k, conv->head_v, s);
        KVT_LAUNCHED("q8_0_to_f16_rows");
    }
    if (n_q > 0 && !host_rows) {   // nothing in host memory
        launch_prefill(q, n_q, q_pos0, n_qh, kvh, group, q_tiles, ph_k, ph_v, n_head,
                       nullptr, nullptr, n_kv, causal, scale, 0, n_kv,
                       n_split > 1 ? stf : nullptr, 1, fin, out, pass_fmt, s, n_split, tps);
        KVT_LAUNCHED("prefill_attn");
    } else if (n_q > 0) {
        bool started = false;
        if (hb > 0) {
            launch_prefill(q, n_q, q_pos0, n_qh, kvh, group, q_tiles, ph_k, ph_v, n_head,
                           nullptr, nullptr, n_kv, causal, scale, 0, hb, stf, 1, 0, out,
                           pass_fmt, s, n_split, tps);
            KVT_LAUNCHED("prefill_attn");
            started = true;
        }
        int b = 0;
        for (int64_t kb = hb; kb < n_kv; kb += slot_keys, b++) {
            const int64_t ke = kb + slot_keys < n_kv ? kb + slot_keys : n_kv;
            const int slot = b & 1;
            const int64_t r0 = kb > n_head ? kb : n_head;   // first host row of the bucket
            const int64_t c0 = b == 0 ? r0 + staged : r0;   // first row this call copies
            const uintptr_t sk = ak + (uintptr_t)(slot * slot_keys * row_bytes);
            const uintptr_t sv = av + (uintptr_t)(slot * slot_keys * row_bytes);
            if (c0 < ke) {
                const size_t bytes = (size_t)(ke - c0) * (size_t)row_bytes;
                const uintptr_t off = (uintptr_t)((c0 - r0) * row_bytes);
                if (b >= 2)
                    KVT_HIP(hipStreamWaitEvent(cs, ev[3 + slot], 0));
                KVT_HIP(hipMemcpyAsync(
                    reinterpret_cast<void *>(sk + off),
                    reinterpret_cast<const void *>(hk + (c0 - n_head) * row_bytes), bytes,
                    hipMemcpyDefault, cs));
                KVT_HIP(hipMemcpyAsync(
                    reinterpret_cast<void *>(sv + off),
                    reinterpret_cast<const void *>(hv + (c0 - n_head) * row_bytes), bytes,
                    hipMemcpyDefault, cs));
                KVT_HIP(hipEventRecord(ev[1 + slot], cs));
                KVT_HIP(hipStreamWaitEvent(s, ev[1 + slot], 0));
            }
            if (b == 0 && staged)
                KVT_HIP(hipStreamWaitEvent(s, ev[5], 0));
            // the kernel reads row r >= n_head at tail + (r - n_head)*row_bytes: aim it at the
            // slot
            uintptr_t tk = sk, tv = sv;
            int64_t trb = row_bytes;
            if (cv) {   // the bucket's rows to fp16; the raw slot is free once they are read
                const uintptr_t ck = reinterpret_cast<uintptr_t>(conv->slot_k) +
                                     (uintptr_t)(slot * slot_keys * row16);
                const uintptr_t cvv = reinterpret_cast<uintptr_t>(conv->slot_v) +
                                      (uintptr_t)(slot * slot_keys * row16);
                convert_rows(reinterpret_cast<const void *>(sk), reinterpret_cast<const void *>(sv),
                             ke - r0, kvh, reinterpret_cast<void *>(ck),
                             reinterpret_cast<void *>(cvv), s);
                KVT_LAUNCHED("q8_0_to_f16_rows");
                KVT_HIP(hipEventRecord(ev[3 + slot], s));
                tk = ck;
                tv = cvv;
                trb = row16;
            }
            const uintptr_t shift = (uintptr_t)((r0 - n_head) * trb);
            launch_prefill(q, n_q, q_pos0, n_qh, kvh, group, q_tiles, ph_k, ph_v, n_head,
                           reinterpret_cast<const void *>(tk - shift),
                           reinterpret_cast<const void *>(tv - shift), n_kv, causal, scale, kb,
                           ke, stf, started ? 0 : 1, ke == n_kv ? fin : 0, out, pass_fmt, s,
                           n_split, tps);
            KVT_LAUNCHED("prefill_attn");
            started = true;
            if (!cv)
                KVT_HIP(hipEventRecord(ev[3 + slot], s));
        }
    }
    if (n_q > 0 && n_split > 1) {
        hipLaunchKernelGGL(prefill_split_merge, dim3((unsigned)(q_tiles * kvh), kWaves), dim3(64),
                           0, s, stf, n_split, (int)kvh, group, n_q, (int)n_qh,
                           (float)((double)scale * 1.4426950408889634), out);
        KVT_LAUNCHED("prefill_split_merge");
    }
    if (prefetch) {   // behind this call's own copies, while its last buckets are attended
        const size_t nb = (size_t)nx.rows * (size_t)row_bytes;
        KVT_HIP(hipMemcpyAsync(reinterpret_cast<void *>(nx.arena_k),
                               reinterpret_cast<const void *>(nx.k_host), nb, hipMemcpyDefault,
                               cs));
        KVT_HIP(hipMemcpyAsync(reinterpret_cast<void *>(nx.arena_v),
                               reinterpret_cast<const void *>(nx.v_host), nb, hipMemcpyDefault,
                               cs));
        KVT_HIP(hipEventRecord(ev[5], cs));
        Prefetched p;
        p.device = dev;
        p.k_host = nx.k_host;
        p.v_host = nx.v_host;
        p.arena_k = nx.arena_k;
        p.arena_v = nx.arena_v;
        p.row_bytes = row_bytes;
        p.rows = nx.rows;
        t_pipe.pre = p;
    }
    return KVT_OK;
}

}  // namespace

// S7+S8 overlapped: the host tail crosses the link in arena-sized buckets on copy_stream while
// stream attends the HBM head and then each staged bucket.
extern "C" int kvt_attn_prefill_pipelined(const void *q, int64_t n_q, int64_t q_pos0,
                                          int32_t n_qh, int32_t kvh, int32_t hd,
                                          const void *k_head, const void *v_head, int64_t n_head,
                                          const void *k_host, const void *v_host, int64_t n_kv,
                                          int32_t kv_format, int32_t causal, float scale,
                                          void *arena_k, void *arena_v, int64_t arena_rows,
                                          void *state, size_t state_bytes_, float *out,
                                          void *stream, void *copy_stream)
{
    return prefill_pipeline("kvt_attn_prefill_pipelined", q, n_q, q_pos0, n_qh, kvh, hd, k_head,
                            v_head, n_head, k_host, v_host, n_kv, kv_format, causal, scale,
                            arena_k, arena_v, arena_rows, 0, NextBucket{}, state, state_bytes_,
                            out, stream, copy_stream);
}

// The same op in a chain of layers: the first `staged_rows` host rows were prefetched by the
// previous call, and the next layer's first `next_rows` host rows are copied into its arena
// behind this call's own copies.
extern "C" int kvt_attn_prefill_chain(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                                      int32_t kvh, int32_t hd, const void *k_head,
                                      const void *v_head, int64_t n_head, const void *k_host,
                                      const void *v_host, int64_t n_kv, int32_t kv_format,
                                      int32_t causal, float scale, void *arena_k, void *arena_v,
                                      int64_t arena_rows, int64_t staged_rows,
                                      const void *next_k_host, const void *next_v_host,
                                      int64_t next_rows, void *next_arena_k, void *next_arena_v,
                                      int64_t next_arena_rows, void *state, size_t state_bytes_,
                                      float *out, void *stream, void *copy_stream)
{
    NextBucket nx;
    nx.k_host = reinterpret_cast<uintptr_t>(next_k_host);
    nx.v_host = reinterpret_cast<uintptr_t>(next_v_host);
    nx.arena_k = reinterpret_cast<uintptr_t>(next_arena_k);
    nx.arena_v = reinterpret_cast<uintptr_t>(next_arena_v);
    nx.rows = next_rows;
    nx.arena_rows = next_arena_rows;
    return prefill_pipeline("kvt_attn_prefill_chain", q, n_q, q_pos0, n_qh, kvh, hd, k_head,
                            v_head, n_head, k_host, v_host, n_kv, kv_format, causal, scale,
                            arena_k, arena_v, arena_rows, staged_rows, nx, state, state_bytes_,
                            out, stream, copy_stream);
}

namespace {

// The auto plan's time model: the host link at the rate contiguous staging copies reach on
// MI355X (56 GB/s), and the prefill kernel's attention rate per cache format when its
// workgroups fill the chip (measured over a 180,000-key cache: q8_0 0.85, fp16 0.98, bf16 0.61
// PFLOP/s).
constexpr double kLinkBytesPerUs = 56.0e3;

double attn_flop_per_us(int32_t fmt)
{
    return fmt == KVT_Q8_0 ? 8.5e8 : fmt == KVT_F16 ? 9.8e8 : 6.1e8;
}

// (query, key) pairs the attention visits: row t sees min(n_kv, q_pos0 + t + 1) keys when
// causal, all n_kv otherwise.
double key_pairs(int64_t n_q, int64_t q_pos0, int64_t n_kv, int32_t causal)
{
    if (!causal)
        return (double)n_q * (double)n_kv;
    int64_t lin = n_kv - q_pos0;   // rows t < lin see q_pos0 + t + 1 keys, the rest n_kv
    lin = lin < 0 ? 0 : (lin > n_q ? n_q : lin);
    const double l = (double)lin;
    return l * (double)(q_pos0 + 1) + l * (l - 1) / 2 + (double)(n_q - lin) * (double)n_kv;
}

}  // namespace

// S7+S8 with the stage-or-read-in-place choice made from the chunk's shape.
extern "C" int kvt_attn_prefill_plan(int64_t n_q, int64_t q_pos0, int32_t n_qh, int32_t kvh,
                                     int64_t n_head, int64_t n_kv, int32_t kv_format,
                                     int32_t causal, int64_t arena_rows, int32_t two_streams)
{
    if (kv_format != KVT_Q8_0 && kv_format != KVT_F16 && kv_format != KVT_BF16)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_prefill_plan: kv_format=%d", kv_format);
    if (kvh < 1 || n_qh < 1 || n_qh % kvh)
        return kvt::fail(KVT_EINVAL, "kvt_attn_prefill_plan: n_qh=%d kvh=%d", n_qh, kvh);
    const int group = n_qh / kvh;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_prefill_plan: group %d", group);
    if (n_q < 0 || q_pos0 < 0 || n_head < 0 || n_head > n_kv || arena_rows < 0)
        return kvt::fail(KVT_EINVAL, "kvt_attn_prefill_plan: n_q=%lld q_pos0=%lld n_head=%lld "
                                     "n_kv=%lld arena_rows=%lld", (long long)n_q,
                         (long long)q_pos0, (long long)n_head, (long long)n_kv,
                         (long long)arena_rows);
    const int64_t tail = n_kv - n_head;
    if (n_q == 0 || tail == 0)
        return KVT_PREFILL_IN_PLACE;   // nothing crosses the link
    const double row_bytes = (double)kvh * head_bytes(kv_format);
    const double stage_us = 2.0 * (double)tail * row_bytes / kLinkBytesPerUs;
    const double attn_us =
        4.0 * kHd * n_qh * key_pairs(n_q, q_pos0, n_kv, causal) / attn_flop_per_us(kv_format);
    const bool fits = arena_rows >= tail;
    // with a second stream and an arena, the copies of one bucket run beside the attention of
    // the last (in key splits when the chunk is short), so the op takes about the longer of
    // the two -- unless the attention is so short (under a quarter of the copy) that hiding
    // it gains less than the extra passes cost, and the whole tail can be staged instead
    if (two_streams && arena_rows / 2 / kKT * kKT >= kKT)
        return fits && 4.0 * attn_us < stage_us ? KVT_PREFILL_STAGED : KVT_PREFILL_PIPELINED;
    // one stream: staged, the tail crosses once at the link rate and then the attention runs;
    // in place, reading scattered head slices takes about twice the copy, beside the
    // attention.  Staging is the shorter when the attention is shorter than the copy.
    return fits && attn_us < stage_us ? KVT_PREFILL_STAGED : KVT_PREFILL_IN_PLACE;
}

// Bytes of the fp16 copies kvt_attn_prefill_auto converts a q8_0 cache's rows into on its
// pipelined plan: the head's n_head rows and the arena's two buckets, K and V.
extern "C" size_t kvt_attn_prefill_conv_bytes(int64_t n_head, int32_t kvh, int64_t arena_rows,
                                              int32_t kv_format)
{
    if (kv_format != KVT_Q8_0 || kvh < 1 || kvh > 240 || n_head < 0 || arena_rows < 0)
        return 0;
    const int64_t slot_keys = arena_rows / 2 / kKT * kKT;
    return (size_t)(2 * (n_head + 2 * slot_keys) * (int64_t)kvh * kHd * 2);
}

extern "C" size_t kvt_attn_prefill_auto_ws_bytes(int64_t n_q, int32_t n_qh, int32_t kvh,
                                                 int64_t n_kv)
{
    const size_t a = kvt_attn_prefill_splitk_ws_bytes(n_q, n_qh, kvh, n_kv);
    const size_t b = kvt_attn_prefill_state_bytes(n_q, n_qh, kvh);
    return a > b ? a : b;
}

extern "C" int kvt_attn_prefill_auto(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                                     int32_t kvh, int32_t hd, const void *k_head,
                                     const void *v_head, int64_t n_head, const void *k_host,
                                     const void *v_host, int64_t n_kv, int32_t kv_format,
                                     int32_t causal, float scale, void *arena_k, void *arena_v,
                                     int64_t arena_rows, void *ws, size_t ws_bytes, void *conv,
                                     size_t conv_bytes, float *out, int32_t *plan, void *stream,
                                     void *copy_stream)
{
    int group = 0;
    int64_t q_tiles = 0;
    int rc = check_prefill("kvt_attn_prefill_auto", q, n_q, q_pos0, n_qh, kvh, hd, k_head,
                           v_head, n_head, k_host, v_host, n_kv, kv_format, scale, out, group,
                           q_tiles);
    if (rc != KVT_OK)
        return rc;
    const bool arena = arena_k && arena_v;
    const bool two = kvt::as_stream(stream) != kvt::as_stream(copy_stream);
    const int p = kvt_attn_prefill_plan(n_q, q_pos0, n_qh, kvh, n_head, n_kv, kv_format, causal,
                                        arena ? arena_rows : 0, two ? 1 : 0);
    if (p < 0)
        return p;
    if (plan)
        *plan = p;
    if (n_q == 0)
        return KVT_OK;
    const int64_t tail = n_kv - n_head;
    if (p == KVT_PREFILL_PIPELINED) {   // in key splits when the chunk is short
        // q8_0: convert every row to fp16 once (the head here, each bucket as it lands) and
        // run the passes on the fp16 kernel -- when the buffer is given and the modelled
        // attention outlasts the conversion (the cache's bytes moved once more at ~4 TB/s).
        // The fp16 passes gain more than the kernels' full-range rates suggest (13%): split over
        // keys, each q8_0 pass pays its raw-tile start again.  Measured at 180,000 keys with a
        // 2 x 16,384-row arena, the conversion won at every chunk from 128 to 2048 queries
        // (512: 4.01 against 4.83 ms).
        Conv cvb;
        const size_t need = kvt_attn_prefill_conv_bytes(n_head, kvh, arena_rows, kv_format);
        if (need && conv && conv_bytes >= need && kvt::aligned(conv, 16)) {
            const double row_bytes = (double)kvh * head_bytes(kv_format);
            const double conv_us = (double)n_kv * 2.0 * (row_bytes + kvh * kHd * 2) / 4.0e6;
            const double attn_us = 4.0 * kHd * n_qh * key_pairs(n_q, q_pos0, n_kv, causal) /
                                   attn_flop_per_us(kv_format);
            if (attn_us > conv_us) {
                const int64_t slot_keys = arena_rows / 2 / kKT * kKT;
                const int64_t row16 = (int64_t)kvh * kHd * 2;
                unsigned char *c = static_cast<unsigned char *>(conv);
                cvb.head_k = c;
                cvb.head_v = c + n_head * row16;
                cvb.slot_k = c + 2 * n_head * row16;
                cvb.slot_v = cvb.slot_k + 2 * slot_keys * row16;
            }
        }
        return prefill_pipeline("kvt_attn_prefill_auto", q, n_q, q_pos0, n_qh, kvh, hd, k_head,
                                v_head, n_head, k_host, v_host, n_kv, kv_format, causal, scale,
                                arena_k, arena_v, arena_rows, 0, NextBucket{}, ws, ws_bytes, out,
                                stream, copy_stream, true, &cvb);
    }
    const void *kt = k_host, *vt = v_host;
    if (p == KVT_PREFILL_STAGED) {
        const int64_t row_bytes = (int64_t)kvh * head_bytes(kv_format);
        rc = kvt_stage_tail(k_host, row_bytes, 0, tail, arena_k, KVT_COPY_AUTO, stream);
        if (rc == KVT_OK)
            rc = kvt_stage_tail(v_host, row_bytes, 0, tail, arena_v, KVT_COPY_AUTO, stream);
        if (rc != KVT_OK)
            return rc;
        kt = arena_k;
        vt = arena_v;
    }
    return kvt_attn_prefill_splitk(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, kt, vt,
                                   n_kv, kv_format, causal, scale, ws, ws_bytes, out, stream);
}
