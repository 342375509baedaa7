// kvt_decode.hip -- S6 GQA decode attention over gathered K/V (split-K, deterministic merge).
//
// QSA-KVO qsa_sparse_attend_rows_staged: query head i reads KV head i / group; each key chunk
// yields a partial (o, m, l) and the partials are folded with the online-softmax rule
// (m' = max, alpha = e^(m - m'), beta = e^(m_c - m'), a chunk with m = -inf contributes 0).
//
// decode_partial: one wavefront per (64-key chunk, KV head, block of four query rows).  All of
//   the chunk's K (as MFMA B operands, straight from HBM) and V (staged in LDS) loads are
//   issued up front, sub-tile by sub-tile.  The group's query heads (padded to 16 rows) times
//   K^T run on v_mfma_f32_16x16x32_{bf16,f16}: bf16/f16 products are exact in fp32,
//   accumulation is fp32.  Softmax and P*V stay in fp32 on the vector ALUs: with at most 16
//   query rows per KV head the PV product is tiny, and keeping the probabilities in fp32 avoids
//   rounding them to 16 bits.
// decode_merge: one thread per (query head, dim) folds the chunks in index order: the global
//   max first, then every chunk rescaled by e^(m_c - max) -- the same fold, one rescale each.
//   One row issues all its loads before the max is reduced (one memory round trip for the
//   step's 32 chunks); many rows stream (decode_merge_rows), with the same arithmetic.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "kvt_internal.h"

namespace {

constexpr int kHd = 128;
constexpr int kKeys = 64;   // keys per chunk (4 MFMA column tiles of 16)
constexpr int kVPitch = kHd * 2 + 4;  // bytes per staged V row (padded)
constexpr int kKPitch = kHd * 2 + 16; // bytes per staged K row (padded, 16-byte aligned)

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

// Online softmax over one 64-key chunk, taken as four 16-key sub-tiles (MFMA column tiles).
// Per query row r of the group: m = running max (log2 domain), l = running sum of 2^(s - m),
// o = running sum of 2^(s - m) v over this lane's two dims.  Sub-tile t: S = Q K_t^T on MFMA,
// keys that take no part masked, m' = max(m, tile max), alpha = 2^(m - m'), then
// l = alpha l + sum 2^(s - m'), o = alpha o + sum 2^(s - m') v.  The staged and the fused
// kernels both run exactly this arithmetic, so they agree bit for bit.
struct ChunkState {
    float m[4], l[4];   // rows 4g + i (replicated over the 16 lanes of group g)
    float o[16][2];     // rows 0..15, dims 2*lane, 2*lane + 1
};

__device__ __forceinline__ void state_init(ChunkState &st)
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        st.m[i] = -INFINITY;
        st.l[i] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; r++)
        st.o[r][0] = st.o[r][1] = 0.f;
}

// The value lane ^ off holds, for off = 1, 2, 4, 8 (inside a row of 16 lanes), by DPP: quad
// permutes for 1 and 2, row shifts up or down by off for 4 and 8.  The same values as
// __shfl_xor, without the LDS permute and its latency.
__device__ __forceinline__ float xor16(float v, int off, int lane)
{
    const int x = __builtin_bit_cast(int, v);
    int r;
    switch (off) {
    case 1: r = __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false); break;   // [1,0,3,2]
    case 2: r = __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false); break;   // [2,3,0,1]
    case 4: {
        const int up = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0xF, false);  // lane + 4
        const int dn = __builtin_amdgcn_update_dpp(x, x, 0x114, 0xF, 0xF, false);  // lane - 4
        r = (lane & 4) ? dn : up;
        break;
    }
    default: {
        const int up = __builtin_amdgcn_update_dpp(x, x, 0x108, 0xF, 0xF, false);  // lane + 8
        const int dn = __builtin_amdgcn_update_dpp(x, x, 0x118, 0xF, 0xF, false);  // lane - 8
        r = (lane & 8) ? dn : up;
        break;
    }
    }
    return __builtin_bit_cast(float, r);
}

// kb: sub-tile t's K as MFMA B operands (lane (g, col): key 16t + col, dims ks*32 + 8g ..);
// vs: the chunk's V rows in LDS; ps [16][16] and as [16]: per-sub-tile LDS scratch.  The output
// rows kept (rescaled and accumulated) are the blocks of four [4*q4_lo, 4*q4_hi); every row's
// arithmetic is its own, so a wave may keep a part of the group's rows.
template <bool kBf16>
__device__ __forceinline__ void subtile_attend(int t, const uint4 (&qa)[4], const uint4 (&kb)[4],
                                               uint64_t valid, int group, float scale_log2,
                                               const unsigned char *vs, float (*ps)[16],
                                               float *as, ChunkState &st, int lane,
                                               int q4_lo = 0, int q4_hi = 4)
{
    const int g = lane >> 4, col = lane & 15;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
        s = mfma16x16x32<kBf16>(qa[ks], kb[ks], s);
    // lane holds S[row 4g+i][key 16t + col]
    const bool ok = (valid >> (16 * t + col)) & 1;
    float mt[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        s[i] = ok ? s[i] * scale_log2 : -INFINITY;
        mt[i] = s[i];
    }
    // row max / sum across the 16 lanes of a group (xor offsets stay inside the group)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
        for (int i = 0; i < 4; i++)
            mt[i] = fmaxf(mt[i], xor16(mt[i], off, lane));
    float alpha[4], ls[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float mn = fmaxf(st.m[i], mt[i]);
        alpha[i] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m[i] - mn);
        const float p = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[i] - mn);
        ps[col][4 * g + i] = p;
        ls[i] = p;
        st.m[i] = mn;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
        for (int i = 0; i < 4; i++)
            ls[i] += xor16(ls[i], off, lane);
#pragma unroll
    for (int i = 0; i < 4; i++)
        st.l[i] = fmaf(st.l[i], alpha[i], ls[i]);
    if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            as[4 * g + i] = alpha[i];
    }
    __syncthreads();   // ps, as visible to the whole wave

    const int nq4 = min((group + 3) >> 2, q4_hi);   // float4 groups of rows kept
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
        if (q4 >= q4_lo && q4 < nq4) {
            const float4 a = *reinterpret_cast<const float4 *>(&as[4 * q4]);
            const float ar[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                st.o[4 * q4 + e][0] *= ar[e];
                st.o[4 * q4 + e][1] *= ar[e];
            }
        }
    }
    // P*V: the sub-tile's 16 V pairs of this lane's two dims, and eight keys' probability vectors
    // of a row block at a time, are read before the FMAs that use them (a read per FMA group
    // would wait on LDS each time); every output still sums its keys in order.
    uint32_t pair[16];
#pragma unroll
    for (int key = 0; key < 16; key++)
        pair[key] = *reinterpret_cast<const uint32_t *>(vs + (16 * t + key) * kVPitch + lane * 4);
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
        if (q4 >= q4_lo && q4 < nq4) {
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 8) {
                float4 p[8];
#pragma unroll
                for (int kk = 0; kk < 8; kk++)
                    p[kk] = *reinterpret_cast<const float4 *>(&ps[k0 + kk][4 * q4]);
#pragma unroll
                for (int kk = 0; kk < 8; kk++) {
                    const float v0 = to_f32((uint16_t)(pair[k0 + kk] & 0xffff), kBf16);
                    const float v1 = to_f32((uint16_t)(pair[k0 + kk] >> 16), kBf16);
                    const float pr[4] = {p[kk].x, p[kk].y, p[kk].z, p[kk].w};
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        st.o[4 * q4 + e][0] = fmaf(pr[e], v0, st.o[4 * q4 + e][0]);
                        st.o[4 * q4 + e][1] = fmaf(pr[e], v1, st.o[4 * q4 + e][1]);
                    }
                }
            }
        }
    }
}

// the chunk's partial (o, m, l) for the group's query rows [4*q4_lo, 4*q4_hi)
__device__ __forceinline__ void write_partial(const ChunkState &st, int group, float *pb,
                                              int lane, int q4_lo = 0, int q4_hi = 4)
{
    const int g = lane >> 4, col = lane & 15;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        if (r < group && r >= 4 * q4_lo && r < 4 * q4_hi)
            *reinterpret_cast<float2 *>(pb + r * (kHd + 2) + 2 * lane) =
                make_float2(st.o[r][0], st.o[r][1]);
    }
    if (col == 0 && g >= q4_lo && g < q4_hi) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = 4 * g + i;
            if (r < group) {
                pb[r * (kHd + 2) + kHd] = st.m[i];
                pb[r * (kHd + 2) + kHd + 1] = st.l[i];
            }
        }
    }
}

// The group's query rows as MFMA A operands (row col of the 16-row tile; rows >= group zero).
__device__ __forceinline__ void load_q(const uint16_t *__restrict__ q, int h, int group, int lane,
                                       uint4 (&qa)[4])
{
    const int g = lane >> 4, col = lane & 15;
    const int qrow = col < group ? col : group - 1;
    const uint16_t *qh = q + ((int64_t)h * group + qrow) * kHd + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
        qa[ks] = *reinterpret_cast<const uint4 *>(qh + ks * 32);
}

// part layout: [kvh][n_chunks][group][kHd + 2]  (o[kHd], m, l); m, l in the log2 domain.
// grid = (chunks, kvh, ceil(group / 4)): the query rows of a KV head are split over waves in
// blocks of four (each wave loads the chunk's K and V, the later ones from L2), which divides
// the VALU work of the PV product -- the wave's critical path once its loads have landed.
template <bool kBf16>
__global__ __launch_bounds__(64) void decode_partial(const uint16_t *__restrict__ q, int group,
                                                     const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v, int64_t n_kv,
                                                     const int32_t *__restrict__ n_valid,
                                                     float scale_log2, float *__restrict__ part)
{
    __shared__ __align__(16) unsigned char vs[kKeys * kVPitch];
    __shared__ __align__(16) float ps[16][16];   // a sub-tile's probabilities, key-major
    __shared__ __align__(16) float as[16];       // a sub-tile's rescale factors per row
    const int lane = threadIdx.x;
    const int c = blockIdx.x, h = blockIdx.y, n_chunks = gridDim.x, q4 = blockIdx.z;
    const int64_t key0 = (int64_t)c * kKeys;
    const int g = lane >> 4, col = lane & 15;

    // Every load below is unconditional, from a clamped (always valid) address, so all of them
    // are in flight together; out-of-range rows are zeroed or masked afterwards.  They are issued
    // sub-tile by sub-tile (its K operands, then its V rows), so a sub-tile is attended as soon as
    // its own loads have landed while the later ones are still in flight (loads complete in issue
    // order for the wait counter); the query and n_valid go first for the same reason.
    uint4 qa[4];
    load_q(q, h, group, lane, qa);
    int64_t nv = n_valid ? (int64_t)n_valid[h] : n_kv;
    const uint16_t *kh = k + (int64_t)h * n_kv * kHd;
    const uint16_t *vh = v + (int64_t)h * n_kv * kHd;
    uint4 kb[4][4];
    uint4 vr[16];
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
        const int64_t key = min(key0 + nt * 16 + col, n_kv - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            kb[nt][ks] = *reinterpret_cast<const uint4 *>(kh + key * kHd + ks * 32 + 8 * g);
#pragma unroll
        for (int j = 4 * nt; j < 4 * nt + 4; j++) {   // V rows 16 nt .. 16 nt + 15
            const int w = lane + 64 * j, row = w >> 4, cw = w & 15;
            const int64_t vkey = min(key0 + row, n_kv - 1);
            vr[j] = *reinterpret_cast<const uint4 *>(vh + vkey * kHd + cw * 8);
        }
    }
    nv = nv < n_kv ? nv : n_kv;
    if (col >= group) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            qa[ks] = make_uint4(0, 0, 0, 0);
    }
    const int64_t nvc = nv - key0;   // keys of this chunk that take part: the first nvc
    const uint64_t valid = nvc >= kKeys ? ~0ull : nvc <= 0 ? 0ull : (1ull << nvc) - 1;
    ChunkState st;
    state_init(st);
#pragma unroll
    for (int t = 0; t < 4; t++) {
        // V rows of keys that take no part are zeroed: their probability is 0, but 0 * NaN is
        // not (rows past n_valid may hold anything, e.g. slots a gather skipped)
#pragma unroll
        for (int j = 4 * t; j < 4 * t + 4; j++) {
            const int w = lane + 64 * j, row = w >> 4, cw = w & 15;
            const uint4 val = key0 + row < nv ? vr[j] : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(vs + row * kVPitch + cw * 16) = val;
        }
        __syncthreads();   // the sub-tile's V rows / the previous sub-tile's ps, as reads are done
        subtile_attend<kBf16>(t, qa, kb[t], valid, group, scale_log2, vs, ps, as, st, lane, q4,
                              q4 + 1);
    }
    write_partial(st, group, part + ((int64_t)h * n_chunks + c) * group * (kHd + 2), lane, q4,
                  q4 + 1);
}

// How a selected slot id becomes the byte offset of its block (token_stride apart rows).
struct SlotMap {
    const int32_t *table;   // NULL: slot id = block index
    int64_t n_ids;          // ids lie in [0, n_ids)
    int64_t n_phys;         // mapped blocks lie in [0, n_phys)
    int64_t block_stride;
    int table_page;         // slots per table entry
    int table_cols;         // entries of the table (row)
    int logical;            // nonzero: the table only validates; the block index stays the id
};

// A slot id's table entry (the load), kept apart from its use so that a loop can issue it
// early.  in: the id lies in [0, n_ids) and its table page in the table.
__device__ __forceinline__ int32_t table_entry(int64_t id, const SlotMap &sm, uint32_t &pg,
                                               bool &in)
{
    in = id >= 0 && id < sm.n_ids;
    const uint32_t u = in ? (uint32_t)id : 0u;
    pg = u / (uint32_t)sm.table_page;
    in = in && (int)pg < sm.table_cols;
    return sm.table ? sm.table[in ? pg : 0] : 0;
}

// slot id (+ its table entry) -> block byte offset, or -1 when the slot takes no part
__device__ __forceinline__ int64_t slot_offset_from(int64_t id, bool in, uint32_t pg,
                                                    int32_t entry, const SlotMap &sm)
{
    bool ok = in;
    if (sm.table) {
        const int64_t phys = entry;
        ok = ok && phys >= 0;
        const int64_t blk =
            phys * sm.table_page + (int64_t)((uint32_t)id - pg * (uint32_t)sm.table_page);
        ok = ok && blk < sm.n_phys;
        if (!sm.logical)
            id = blk;
    }
    return ok ? id * sm.block_stride : -1;
}

__device__ __forceinline__ int64_t slot_offset(int64_t id, const SlotMap &sm)
{
    uint32_t pg;
    bool in;
    const int32_t e = table_entry(id, sm, pg, in);
    return slot_offset_from(id, in, pg, e, sm);
}

// Gather and attend one 64-key chunk: the chunk's K/V rows are read straight from the
// (host-mapped) planes of the selected slots, optionally written to the HBM gather buffers,
// and folded into st.  Key j (j < kk*bt) is token j % bt of selected slot j / bt.  Each lane
// owns the 16-byte word cw = lane % 16 of rows lane/16 + 4*jj (jj < 16): every group of 16
// lanes reads one contiguous 256-byte row slice.
//   sbase: lane L's block offset of slot s0 + L (s0 = key0 / bt), from slot_offset;
//   mid(): called once the chunk's first row loads are issued (a loop prefetches there).
template <bool kBf16, bool kPaced, typename Mid>
__device__ __forceinline__ void gather_chunk(
    const unsigned char *__restrict__ kp, const unsigned char *__restrict__ vp, int64_t sbase,
    int64_t hoff, int64_t token_stride, int bt, int kk, int key0, uint16_t *__restrict__ k_out,
    uint16_t *__restrict__ v_out, int64_t out_key0, uint4 (&qa)[4], int group,
    float scale_log2, unsigned char *ksm, unsigned char *vs, float (*ps)[16], float *as,
    ChunkState &st, int lane, Mid mid)
{
    const int n_kv = kk * bt;   // < 2^31, checked by the host
    const int rg = lane >> 4, cw = lane & 15;
    const int s0 = (int)((uint32_t)key0 / (uint32_t)bt);
    // byte offsets of this lane's 16 rows (cw*16 -- always a valid address -- for keys that
    // take no part); bit jj of okb = row rg + 4*jj takes part
    int slot[16];
    int64_t base[16];
#pragma unroll
    for (int jj = 0; jj < 16; jj++) {
        const int key = key0 + rg + 4 * jj;
        slot[jj] = (int)((uint32_t)(key < n_kv ? key : n_kv - 1) / (uint32_t)bt);
    }
#pragma unroll
    for (int jj = 0; jj < 16; jj++)
        base[jj] = __shfl(sbase, slot[jj] - s0, 64);
    int64_t off[16];
    uint32_t okb = 0;
#pragma unroll
    for (int jj = 0; jj < 16; jj++) {
        const int key = key0 + rg + 4 * jj;
        const int r = (key < n_kv ? key : n_kv - 1) - slot[jj] * bt;
        const bool ok = key < n_kv && base[jj] >= 0;
        off[jj] = ok ? base[jj] + hoff + (int64_t)r * token_stride : (int64_t)cw * 16;
        okb |= (uint32_t)ok << jj;
    }
    // keys that take part, as a chunk bit mask (lanes 0, 16, 32, 48 own rows 4jj + 0..3)
    uint64_t valid = 0;
#pragma unroll
    for (int jj = 0; jj < 16; jj++) {
        const uint64_t bal = __ballot((okb >> jj) & 1);
        valid |= ((bal & 1) | ((bal >> 15) & 2) | ((bal >> 30) & 4) | ((bal >> 45) & 8)) << (4 * jj);
    }
    // query rows past the group are zero (here, not at their load: that would make the id and
    // row loads above wait for the query loads)
    if ((lane & 15) >= group) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            qa[ks] = make_uint4(0, 0, 0, 0);
    }
    // Paced (planes across the host link): the rows cross the link one K and one V wave-load
    // at a time per wave -- with every load of the step issued at once the link runs ~20%
    // slower (see kvt_gather.hip) -- and the pair after a sub-tile's last is issued before
    // that sub-tile is attended, so the attention runs while the link is busy.  Each pair
    // goes to LDS -- K as read, V zeroed where the key takes no part -- and, when asked, to
    // the HBM gather buffers in kvt_gather_blocks' layout (rows of skipped slots untouched).
    // Unpaced (planes in HBM): every load of the chunk is issued at once.
    if constexpr (!kPaced) {
        // HBM planes: K straight into the MFMA B layout (lane (g, col) takes key 16t + col,
        // dims ks*32 + 8g ..), V rows through LDS as below; no K staging in LDS, so twice as
        // many waves fit a CU.  A key that takes no part reads the plane's first bytes; its
        // scores are masked.
        const int g = lane >> 4, col = lane & 15;
        const int64_t hk = hoff - cw * 16;   // the head's offset inside a row
        uint4 kd[4][4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int key = key0 + 16 * t + col;
            const int kc = key < n_kv ? key : n_kv - 1;
            const int sl = (int)((uint32_t)kc / (uint32_t)bt);
            const int64_t b = __shfl(sbase, sl - s0, 64);
            const bool ok = key < n_kv && b >= 0;
            const int64_t o = ok ? b + hk + (int64_t)(kc - sl * bt) * token_stride + 16 * g : 0;
#pragma unroll
            for (int ks = 0; ks < 4; ks++)
                kd[t][ks] = *reinterpret_cast<const uint4 *>(kp + o + ks * 64);
        }
        u32x4 vr[16];
#pragma unroll
        for (int jj = 0; jj < 16; jj++)
            vr[jj] = *reinterpret_cast<const u32x4 *>(vp + off[jj]);
        mid();
#pragma unroll
        for (int t = 0; t < 4; t++) {
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int jj = 4 * t + u;
                *reinterpret_cast<u32x4 *>(vs + (rg + 4 * jj) * kVPitch + cw * 16) =
                    ((okb >> jj) & 1) ? vr[jj] : u32x4{0, 0, 0, 0};
            }
            __syncthreads();   // sub-tile t's V rows are in LDS
            subtile_attend<kBf16>(t, qa, kd[t], valid, group, scale_log2, vs, ps, as, st, lane);
        }
        return;
    }
    u32x4 kr[1], vr[1];
    kr[0] = *reinterpret_cast<const u32x4 *>(kp + off[0]);
    vr[0] = *reinterpret_cast<const u32x4 *>(vp + off[0]);
    mid();
#pragma unroll
    for (int t = 0; t < 4; t++) {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int jj = 4 * t + u;
            const int row = rg + 4 * jj;
            const bool ok = (okb >> jj) & 1;
            const u32x4 kx = kr[0], vx = vr[0];
            *reinterpret_cast<u32x4 *>(ksm + row * kKPitch + cw * 16) = kx;
            *reinterpret_cast<u32x4 *>(vs + row * kVPitch + cw * 16) =
                ok ? vx : u32x4{0, 0, 0, 0};
            if (k_out && ok) {
                const int64_t e = (out_key0 + key0 + row) * kHd + cw * 8;
                *reinterpret_cast<u32x4 *>(k_out + e) = kx;
                *reinterpret_cast<u32x4 *>(v_out + e) = vx;
            }
            __asm__ volatile("" ::: "memory");   // keep the next pair behind this one
            if (jj + 1 < 16) {
                kr[0] = *reinterpret_cast<const u32x4 *>(kp + off[jj + 1]);
                vr[0] = *reinterpret_cast<const u32x4 *>(vp + off[jj + 1]);
            }
        }
        __syncthreads();   // sub-tile t's K and V rows are in LDS
        // K as MFMA B operands: lane (g, col) takes key 16t + col, dims ks*32 + 8g .. +7
        const int g = lane >> 4, col = lane & 15;
        uint4 kb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
            kb[ks] = *reinterpret_cast<const uint4 *>(ksm + (16 * t + col) * kKPitch + ks * 64 +
                                                      16 * g);
        subtile_attend<kBf16>(t, qa, kb, valid, group, scale_log2, vs, ps, as, st, lane);
    }
}

// grid = (splits, kvh, rows); split x of row z, KV head y folds chunks
// [x*chunks_per_wg, min((x+1)*chunks_per_wg, n_chunks)) of that row's keys.
//   q: [rows][kvh*group][kHd];  ids of (row, head): ids + row*ids_row_stride + h*ids_head_stride;
//   table (row): sm.table + row*table_row_stride;  part: [rows][kvh][splits][group][kHd + 2].
// kLoop false: one chunk per workgroup (chunks_per_wg == 1), straight-line code -- the decode
// step, the only form that writes k_out/v_out.  kPaced: see gather_chunk.
template <bool kBf16, bool kLoop, bool kPaced>
__global__ __launch_bounds__(64) void gather_decode_partial(
    const uint16_t *__restrict__ q, int group, const unsigned char *__restrict__ kp,
    const unsigned char *__restrict__ vp, SlotMap sm, int64_t head_stride, int64_t token_stride,
    int64_t table_row_stride, int bt, const int32_t *__restrict__ ids, int64_t ids_row_stride,
    int ids_head_stride, int kk, int chunks_per_wg, uint16_t *__restrict__ k_out,
    uint16_t *__restrict__ v_out, float scale_log2, float *__restrict__ part)
{
    __shared__ __align__(16) unsigned char ksm[kPaced ? kKeys * kKPitch : 16];   // unpaced: unused
    __shared__ __align__(16) unsigned char vs[kKeys * kVPitch];
    __shared__ __align__(16) float ps[16][16];
    __shared__ __align__(16) float as[16];
    const int lane = threadIdx.x;
    const int x = blockIdx.x, h = blockIdx.y, row = blockIdx.z, n_split = gridDim.x;
    const int kvh = gridDim.y;
    const int n_chunks = (kk * bt + kKeys - 1) / kKeys;
    const int cw = lane & 15;

    // the query rows first: their loads must not queue behind the host reads
    uint4 qa[4];
    load_q(q + (int64_t)row * kvh * group * kHd, h, group, lane, qa);
    const int32_t *hid = ids + (int64_t)row * ids_row_stride + (int64_t)h * ids_head_stride;
    SlotMap rsm = sm;
    if (rsm.table)
        rsm.table += (int64_t)row * table_row_stride;
    const int64_t hoff = (int64_t)h * head_stride + cw * 16;
    ChunkState st;
    state_init(st);
    if constexpr (kLoop) {
        // Chunk c + 1's ids are loaded before chunk c's rows and its table entries right after
        // them, so neither lookup waits in line in front of the next chunk's row loads.
        const int c0 = x * chunks_per_wg, c1 = min(c0 + chunks_per_wg, n_chunks);
        const int n_kv = kk * bt;
        int64_t id = hid[min((int)((uint32_t)(c0 * kKeys) / (uint32_t)bt) + lane, kk - 1)];
        uint32_t pg;
        bool in;
        int32_t ent = table_entry(id, rsm, pg, in);
        for (int c = c0; c < c1; c++) {
            if (c != c0)
                __syncthreads();   // the previous chunk's LDS rows are no longer read
            const int64_t sbase = slot_offset_from(id, in, pg, ent, rsm);
            const bool more = c + 1 < c1;
            const int s1 = (int)((uint32_t)min((c + 1) * kKeys, n_kv - 1) / (uint32_t)bt);
            const int64_t id_n = hid[min(s1 + lane, kk - 1)];
            uint32_t pg_n = 0;
            bool in_n = false;
            int32_t ent_n = 0;
            gather_chunk<kBf16, kPaced>(kp, vp, sbase, hoff, token_stride, bt, kk, c * kKeys,
                                        nullptr, nullptr, 0, qa, group, scale_log2, ksm, vs, ps,
                                        as, st, lane, [&] {
                                            if (more)
                                                ent_n = table_entry(id_n, rsm, pg_n, in_n);
                                        });
            id = id_n;
            pg = pg_n;
            in = in_n;
            ent = ent_n;
        }
    } else {
        const int s0 = (int)((uint32_t)(x * kKeys) / (uint32_t)bt);
        const int64_t sbase = slot_offset(hid[min(s0 + lane, kk - 1)], rsm);
        gather_chunk<kBf16, kPaced>(kp, vp, sbase, hoff, token_stride, bt, kk, x * kKeys, k_out,
                                    v_out, (int64_t)h * kk * bt, qa, group, scale_log2, ksm, vs,
                                    ps, as, st, lane, [] {});
    }
    write_partial(st, group,
                  part + (((int64_t)row * kvh + h) * n_split + x) * group * (kHd + 2), lane);
}

// grid = (n_qh, 1), block = kHd (one row: few workgroups, latency-bound).  The global max of the
// chunks' m, then the weighted sums in chunk order: deterministic.  Every load of the first
// kMergeBatch chunks (this thread's output element of each, the m and l of chunk threadIdx.x)
// is issued before the max is reduced, so up to kMergeBatch chunks take one memory round trip;
// the weights and l's of a batch of kHd chunks go through LDS.
constexpr int kMergeBatch = 32;
__global__ __launch_bounds__(kHd) void decode_merge(const float *__restrict__ part, int group,
                                                    int n_chunks, float *__restrict__ out)
{
    __shared__ float s_w[kHd], s_l[kHd], s_max[kHd / 64];
    const int qh = blockIdx.x, d = threadIdx.x, n_qh = gridDim.x;
    const int h = qh / group, r = qh % group;
    part += (int64_t)blockIdx.y * n_qh * n_chunks * (kHd + 2);
    out += (int64_t)blockIdx.y * n_qh * kHd;
    if (n_chunks <= 0) {
        out[(int64_t)qh * kHd + d] = 0.f;
        return;
    }
    const float *base = part + ((int64_t)h * n_chunks * group + r) * (kHd + 2);
    const int64_t cstride = (int64_t)group * (kHd + 2);
    // the loads past the last chunk are skipped (a uniform condition); the empty asm takes the
    // values as operands, which keeps the loads here, ahead of the reduction (the compiler
    // would otherwise sink them, read-only as they are, to their uses after the barrier)
    float v[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; j++)
        v[j] = j < n_chunks ? base[j * cstride + d] : 0.f;
    const int cd = min(d, n_chunks - 1);
    float mc = base[cd * cstride + kHd], lc = base[cd * cstride + kHd + 1];
#pragma unroll
    for (int j = 0; j < kMergeBatch; j++)
        asm volatile("" : "+v"(v[j]));
    if (d >= n_chunks) {
        mc = -INFINITY;
        lc = 0.f;
    }
    float M = fmaxf(-INFINITY, mc);
    for (int c = d + kHd; c < n_chunks; c += kHd)
        M = fmaxf(M, base[c * cstride + kHd]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        M = fmaxf(M, __shfl_xor(M, o, 64));
    if ((d & 63) == 0)
        s_max[d >> 6] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kHd / 64; w++)
        M = fmaxf(M, s_max[w]);
    float acc = 0.f, l = 0.f;
    if (M != -INFINITY) {
        for (int c0 = 0; c0 < n_chunks; c0 += kHd) {
            const int c = c0 + d;
            if (c0 > 0) {
                mc = -INFINITY;
                lc = 0.f;
                if (c < n_chunks) {
                    mc = base[c * cstride + kHd];
                    lc = base[c * cstride + kHd + 1];
                }
            }
            s_w[d] = c < n_chunks && mc != -INFINITY ? __builtin_amdgcn_exp2f(mc - M) : 0.f;
            s_l[d] = lc;
            __syncthreads();
            const int nb = min(kHd, n_chunks - c0);
            for (int j0 = 0; j0 < nb; j0 += kMergeBatch) {
                if (c0 + j0 > 0) {
#pragma unroll
                    for (int j = 0; j < kMergeBatch; j++)
                        v[j] = j0 + j < nb ? base[(c0 + j0 + j) * cstride + d] : 0.f;
                }
#pragma unroll
                for (int j = 0; j < kMergeBatch; j++)
                    if (j0 + j < nb) {
                        const float w = s_w[j0 + j];
                        acc = fmaf(v[j], w, acc);
                        l = fmaf(s_l[j0 + j], w, l);
                    }
            }
            __syncthreads();
        }
    }
    out[(int64_t)qh * kHd + d] = l > 0.f ? acc / l : 0.f;
}

// grid = (n_qh, rows) with many rows, block = kHd: the same fold as decode_merge in two
// streaming passes over the chunks (global max, then the weighted sums, eight loads in flight),
// with no barrier: many workgroups share each CU, so this form keeps fewer instructions per
// output instead of taking one round trip per workgroup.  Same operations in the same order as
// decode_merge: the two give the same bits.
__global__ __launch_bounds__(kHd) void decode_merge_rows(const float *__restrict__ part, int group,
                                                    int n_chunks, float *__restrict__ out)
{
    const int qh = blockIdx.x, d = threadIdx.x, n_qh = gridDim.x;
    const int h = qh / group, r = qh % group;
    part += (int64_t)blockIdx.y * n_qh * n_chunks * (kHd + 2);
    out += (int64_t)blockIdx.y * n_qh * kHd;
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
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_decode: hd=%d (supported: 128)", hd);
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
        const dim3 grid((unsigned)chunks, kvh, (group + 3) / 4);
        if (dtype == KVT_BF16)
            hipLaunchKernelGGL(decode_partial<true>, grid, dim3(64), 0, s,
                               static_cast<const uint16_t *>(q), group,
                               static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                               n_kv, n_valid, scale_log2, part);
        else
            hipLaunchKernelGGL(decode_partial<false>, grid, dim3(64), 0, s,
                               static_cast<const uint16_t *>(q), group,
                               static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v),
                               n_kv, n_valid, scale_log2, part);
        KVT_LAUNCHED("decode_partial");
    }
    hipLaunchKernelGGL(decode_merge, dim3(n_qh), dim3(kHd), 0, s, part, group, (int)chunks, out);
    KVT_LAUNCHED("decode_merge");
    return KVT_OK;
}

namespace {

// Argument checks shared by the workspace and the no-allocation forms of the fused decode;
// returns KVT_OK and the key count, or the failure status.
int gather_attn_decode_check(const char *who, const void *q, int32_t n_qh, int32_t kvh,
                             int32_t hd, int32_t dtype, const void *k_plane, const void *v_plane,
                             int64_t n_blocks, int64_t block_stride, int64_t head_stride,
                             int64_t token_stride, int32_t bt, const int32_t *ids, int32_t k,
                             const void *k_out, const void *v_out, const float *out,
                             int64_t *n_kv)
{
    if (hd != kHd)
        return kvt::fail(KVT_EUNSUPPORTED, "%s: hd=%d (supported: 128)", who, hd);
    if (dtype != KVT_BF16 && dtype != KVT_F16)
        return kvt::fail(KVT_EUNSUPPORTED, "%s: dtype=%d", who, dtype);
    if (n_qh < 1 || kvh < 1 || n_qh % kvh || n_qh / kvh > 16 || kvh > 65535 || bt < 1 || k < 1 ||
        n_blocks < 1)
        return kvt::fail(KVT_EINVAL, "%s: n_qh=%d kvh=%d bt=%d k=%d n_blocks=%lld", who, n_qh,
                         kvh, bt, k, (long long)n_blocks);
    if ((int64_t)k * bt > 0x7fffffffll - kKeys)
        return kvt::fail(KVT_ERANGE, "%s: k*bt too large", who);
    if (block_stride % 16 || head_stride % 16 || token_stride % 16 || block_stride < 0 ||
        head_stride < 0 || token_stride < 0)
        return kvt::fail(KVT_EALIGN,
                         "%s: strides (%lld, %lld, %lld) must be non-negative multiples of 16",
                         who, (long long)block_stride, (long long)head_stride,
                         (long long)token_stride);
    if (!q || !out || !k_plane || !v_plane || !ids || (!k_out) != (!v_out))
        return kvt::fail(KVT_EINVAL, "%s: null pointer (k_out and v_out are both given or both "
                                     "NULL)", who);
    if (!kvt::aligned(q, 16) || !kvt::aligned(k_plane, 16) || !kvt::aligned(v_plane, 16) ||
        !kvt::aligned(k_out, 16) || !kvt::aligned(v_out, 16))
        return kvt::fail(KVT_EALIGN, "%s: q, planes and outputs must be 16-byte aligned", who);
    *n_kv = (int64_t)k * bt;
    return KVT_OK;
}

// Enqueues the fused gather + attention with its split partials in `part` (checked already).
int gather_attn_decode_launch(const void *q, int32_t n_qh, int32_t kvh, int32_t dtype,
                              const void *k_plane, const void *v_plane, int64_t n_blocks,
                              int64_t block_stride, int64_t head_stride, int64_t token_stride,
                              const int32_t *block_table, int32_t bt, const int32_t *ids,
                              int32_t k, void *k_out, void *v_out, float scale, float *out,
                              float *part, hipStream_t s)
{
    const int64_t n_kv = (int64_t)k * bt;
    const int64_t chunks = (n_kv + kKeys - 1) / kKeys;
    const int group = n_qh / kvh;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    const SlotMap sm{block_table, n_blocks, n_blocks, block_stride, 1,
                     (int)std::min<int64_t>(n_blocks, 0x7fffffff), 0};
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)chunks, kvh, 1), dim3(64), 0, s,
                           static_cast<const uint16_t *>(q), group,
                           static_cast<const unsigned char *>(k_plane),
                           static_cast<const unsigned char *>(v_plane), sm, head_stride,
                           token_stride, (int64_t)0, (int)bt, ids, (int64_t)0, (int)k, (int)k, 1,
                           static_cast<uint16_t *>(k_out), static_cast<uint16_t *>(v_out),
                           scale_log2, part);
    };
    if (dtype == KVT_BF16)
        launch(gather_decode_partial<true, false, true>);
    else
        launch(gather_decode_partial<false, false, true>);
    KVT_LAUNCHED("gather_decode_partial");
    hipLaunchKernelGGL(decode_merge, dim3(n_qh), dim3(kHd), 0, s, part, group, (int)chunks, out);
    KVT_LAUNCHED("decode_merge");
    return KVT_OK;
}

// The no-allocation form's scratch: the split partials live in this fixed array, one copy per
// GPU, held until the process ends.  Host code never passes its name to a kernel (on the host
// the name is a stand-in, not a device address): it uses the address hipGetSymbolAddress
// returns for each device, taken once per device with that device current.
constexpr size_t kNoAllocScratchBytes = 4u << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxScratchDevices] = {};

int scratch_for_device(int dev, void **addr)
{
    if (dev < 0 || dev >= kMaxScratchDevices)
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_gather_attn_decode_noalloc: device %d out of "
                                           "range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        int cur = 0;
        KVT_HIP(hipGetDevice(&cur));
        KVT_HIP(hipSetDevice(dev));
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return kvt::fail(KVT_EHIP, "kvt_gather_attn_decode_noalloc: hipGetSymbolAddress: %s",
                             hipGetErrorString(e));
        if (e2 != hipSuccess)
            return kvt::fail(KVT_EHIP, "kvt_gather_attn_decode_noalloc: hipSetDevice: %s",
                             hipGetErrorString(e2));
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return KVT_OK;
}

}  // namespace

// S5+S6 in one pass: QSA-KVO's decode reads the selected K/V blocks through base pointers and
// computed offsets; here each chunk's rows cross the host link straight into the wave that
// attends them (and, when k_out/v_out are given, into the HBM gather buffers as well).
extern "C" int kvt_gather_attn_decode(const void *q, int32_t n_qh, int32_t kvh, int32_t hd,
                                      int32_t dtype, const void *k_plane, const void *v_plane,
                                      int64_t n_blocks, int64_t block_stride, int64_t head_stride,
                                      int64_t token_stride, const int32_t *block_table, int32_t bt,
                                      const int32_t *ids, int32_t k, void *k_out, void *v_out,
                                      float scale, float *out, void *ws, size_t ws_bytes,
                                      void *stream)
{
    int64_t n_kv = 0;
    const int rc = gather_attn_decode_check("kvt_gather_attn_decode", q, n_qh, kvh, hd, dtype,
                                            k_plane, v_plane, n_blocks, block_stride,
                                            head_stride, token_stride, bt, ids, k, k_out, v_out,
                                            out, &n_kv);
    if (rc != KVT_OK)
        return rc;
    const size_t need = kvt_attn_decode_ws_bytes(n_qh, hd, n_kv);
    if (!ws || ws_bytes < need)
        return kvt::fail(KVT_EINVAL, "kvt_gather_attn_decode: workspace of %zu bytes, need %zu",
                         ws_bytes, need);
    return gather_attn_decode_launch(q, n_qh, kvh, dtype, k_plane, v_plane, n_blocks,
                                     block_stride, head_stride, token_stride, block_table, bt,
                                     ids, k, k_out, v_out, scale, out, static_cast<float *>(ws),
                                     kvt::as_stream(stream));
}

// The same pass for callers that cannot allocate: the partials go to the library's fixed
// per-GPU scratch array instead of a caller workspace (kvt_gather_attn_decode_noalloc in kvt.h).
extern "C" size_t kvt_gather_attn_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int kvt_gather_attn_decode_noalloc(const void *q, int32_t n_qh, int32_t kvh,
                                              int32_t hd, int32_t dtype, const void *k_plane,
                                              const void *v_plane, int64_t n_blocks,
                                              int64_t block_stride, int64_t head_stride,
                                              int64_t token_stride, const int32_t *block_table,
                                              int32_t bt, const int32_t *ids, int32_t k,
                                              void *k_out, void *v_out, float scale, float *out,
                                              void *stream)
{
    int64_t n_kv = 0;
    int rc = gather_attn_decode_check("kvt_gather_attn_decode_noalloc", q, n_qh, kvh, hd, dtype,
                                      k_plane, v_plane, n_blocks, block_stride, head_stride,
                                      token_stride, bt, ids, k, k_out, v_out, out, &n_kv);
    if (rc != KVT_OK)
        return rc;
    const size_t need = kvt_attn_decode_ws_bytes(n_qh, hd, n_kv);
    if (need > kNoAllocScratchBytes)
        return kvt::fail(KVT_ERANGE, "kvt_gather_attn_decode_noalloc: the partials need %zu "
                                     "bytes, more than the %zu-byte scratch (n_qh * "
                                     "ceil(k*bt/64) * 130 * 4 bytes)", need,
                         kNoAllocScratchBytes);
    hipStream_t s = kvt::as_stream(stream);
    int dev = 0;
    KVT_HIP(hipStreamGetDevice(s, &dev));
    void *part = nullptr;
    rc = scratch_for_device(dev, &part);
    if (rc != KVT_OK)
        return rc;
    return gather_attn_decode_launch(q, n_qh, kvh, dtype, k_plane, v_plane, n_blocks,
                                     block_stride, head_stride, token_stride, block_table, bt,
                                     ids, k, k_out, v_out, scale, out, static_cast<float *>(part),
                                     s);
}

// [QSA-KVO] qsa_staging_worthwhile: the direct path reads rows * k_pad positions over the link
// (each row its own selection, overlapping heavily); staging reads each used page once.
extern "C" int kvt_staging_worthwhile(int64_t rows, int64_t k_pad, int64_t pages_used,
                                      int64_t page_size)
{
    if (rows < 0 || k_pad < 0 || pages_used < 0 || page_size < 0)
        return 0;
    return (double)rows * (double)k_pad > 2.0 * (double)pages_used * (double)page_size ? 1 : 0;
}

namespace {

constexpr int kRowsTargetGroups = 2048;   // workgroups to aim for: 8 per CU

// chunks per workgroup and splits for `rows` rows of k_pad positions
void rows_split(int64_t rows, int kvh, int64_t k_pad, int &chunks_per_wg, int &splits)
{
    const int64_t chunks = std::max<int64_t>(1, (k_pad + kKeys - 1) / kKeys);
    int64_t want = (kRowsTargetGroups + rows * kvh - 1) / std::max<int64_t>(1, rows * kvh);
    want = std::max<int64_t>(1, std::min(want, chunks));
    chunks_per_wg = (int)((chunks + want - 1) / want);
    splits = (int)((chunks + chunks_per_wg - 1) / chunks_per_wg);
}

// Both planes in device memory (HBM)?  Reads across the host link are paced; HBM reads are not.
bool in_hbm(const void *a, const void *b)
{
    for (const void *p : {a, b}) {
        hipPointerAttribute_t at;
        if (hipPointerGetAttributes(&at, p) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        if (at.type != hipMemoryTypeDevice)
            return false;
    }
    return true;
}

struct RowsArgs {
    const void *q;
    int32_t rows, n_qh, kvh, hd, dtype;
    const void *k_plane, *v_plane;
    int64_t n_rows, row_stride, head_stride;
    const int32_t *table;
    int32_t table_cols;
    int64_t table_row_stride;
    int32_t page_size;
    const int32_t *positions;
    int32_t k_pad;
    float scale;
    float *out;
    void *ws;
    size_t ws_bytes;
};

int check_rows(const char *fn, const RowsArgs &a)
{
    if (a.hd != kHd)
        return kvt::fail(KVT_EUNSUPPORTED, "%s: hd=%d (supported: 128)", fn, a.hd);
    if (a.dtype != KVT_BF16 && a.dtype != KVT_F16)
        return kvt::fail(KVT_EUNSUPPORTED, "%s: dtype=%d", fn, a.dtype);
    if (a.rows < 0 || a.rows > 65535 || a.n_qh < 1 || a.kvh < 1 || a.n_qh % a.kvh ||
        a.n_qh / a.kvh > 16 || a.kvh > 65535 || a.k_pad < 1 || a.k_pad > 0x7fffffff - kKeys ||
        a.n_rows < 1 || a.n_rows > 0x7fffffffll)
        return kvt::fail(KVT_EINVAL, "%s: rows=%d n_qh=%d kvh=%d k_pad=%d n_rows=%lld", fn,
                         a.rows, a.n_qh, a.kvh, a.k_pad, (long long)a.n_rows);
    if (a.table && (a.page_size < 1 || a.table_cols < 1 || a.table_row_stride < 0))
        return kvt::fail(KVT_EINVAL, "%s: page_size=%d table_cols=%d table_row_stride=%lld", fn,
                         a.page_size, a.table_cols, (long long)a.table_row_stride);
    if (a.row_stride % 16 || a.head_stride % 16 || a.row_stride < 0 || a.head_stride < 0)
        return kvt::fail(KVT_EALIGN, "%s: strides (%lld, %lld) must be non-negative multiples "
                         "of 16", fn, (long long)a.row_stride, (long long)a.head_stride);
    if (a.head_stride * (a.kvh - 1) + (int64_t)a.hd * 2 > a.row_stride)
        return kvt::fail(KVT_EINVAL, "%s: %d heads at stride %lld do not fit a row of %lld bytes",
                         fn, a.kvh, (long long)a.head_stride, (long long)a.row_stride);
    if (!a.q || !a.out || !a.k_plane || !a.v_plane || !a.positions)
        return kvt::fail(KVT_EINVAL, "%s: null pointer", fn);
    if (!kvt::aligned(a.q, 16) || !kvt::aligned(a.k_plane, 16) || !kvt::aligned(a.v_plane, 16))
        return kvt::fail(KVT_EALIGN, "%s: q and planes must be 16-byte aligned", fn);
    const size_t need = kvt_sparse_attend_rows_ws_bytes(a.rows, a.n_qh, a.kvh, a.k_pad);
    if (!a.ws || a.ws_bytes < need)
        return kvt::fail(KVT_EINVAL, "%s: workspace of %zu bytes, need %zu", fn, a.ws_bytes,
                         need);
    return KVT_OK;
}

// the attention over the rows' positions; sm says where a position's row lives
int launch_rows(const char *fn, const RowsArgs &a, const void *kp, const void *vp,
                const SlotMap &sm, bool paced, void *stream)
{
    if (a.rows == 0)
        return KVT_OK;
    int cpw = 1, splits = 1;
    rows_split(a.rows, a.kvh, a.k_pad, cpw, splits);
    hipStream_t s = kvt::as_stream(stream);
    const int group = a.n_qh / a.kvh;
    float *part = static_cast<float *>(a.ws);
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);  // log2(e)
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)splits, a.kvh, a.rows), dim3(64), 0, s,
                           static_cast<const uint16_t *>(a.q), group,
                           static_cast<const unsigned char *>(kp),
                           static_cast<const unsigned char *>(vp), sm, a.head_stride,
                           (int64_t)0, a.table_row_stride, 1, a.positions, (int64_t)a.k_pad, 0,
                           (int)a.k_pad, cpw, (uint16_t *)nullptr, (uint16_t *)nullptr,
                           scale_log2, part);
    };
    const bool bf = a.dtype == KVT_BF16;
    if (paced) {
        if (cpw == 1)
            bf ? launch(gather_decode_partial<true, false, true>)
               : launch(gather_decode_partial<false, false, true>);
        else
            bf ? launch(gather_decode_partial<true, true, true>)
               : launch(gather_decode_partial<false, true, true>);
    } else {
        if (cpw == 1)
            bf ? launch(gather_decode_partial<true, false, false>)
               : launch(gather_decode_partial<false, false, false>);
        else
            bf ? launch(gather_decode_partial<true, true, false>)
               : launch(gather_decode_partial<false, true, false>);
    }
    KVT_LAUNCHED("gather_decode_partial");
    if (a.rows == 1)
        hipLaunchKernelGGL(decode_merge, dim3(a.n_qh, 1), dim3(kHd), 0, s, part, group, splits,
                           a.out);
    else
        hipLaunchKernelGGL(decode_merge_rows, dim3(a.n_qh, a.rows), dim3(kHd), 0, s, part, group,
                           splits, a.out);
    KVT_LAUNCHED("decode_merge");
    (void)fn;
    return KVT_OK;
}

}  // namespace

extern "C" size_t kvt_sparse_attend_rows_ws_bytes(int32_t rows, int32_t n_qh, int32_t kvh,
                                                  int32_t k_pad)
{
    if (rows < 0 || n_qh < 1 || kvh < 1 || k_pad < 1)
        return 0;
    int cpw = 1, splits = 1;
    rows_split(std::max(rows, 1), kvh, k_pad, cpw, splits);
    return (size_t)std::max(rows, 1) * (size_t)n_qh * (size_t)splits * (kHd + 2) * sizeof(float);
}

// [QSA-KVO] qsa_sparse_attend_rows: each query row attends its own selection of cache
// positions, read in place (host-mapped or HBM planes) through the row's page table.
extern "C" int kvt_sparse_attend_rows(const void *q, int32_t rows, int32_t n_qh, int32_t kvh,
                                      int32_t hd, int32_t dtype, const void *k_plane,
                                      const void *v_plane, int64_t n_rows, int64_t row_stride,
                                      int64_t head_stride, const int32_t *block_table,
                                      int32_t table_cols, int64_t table_row_stride,
                                      int32_t page_size, const int32_t *positions, int32_t k_pad,
                                      float scale, float *out, void *ws, size_t ws_bytes,
                                      void *stream)
{
    const RowsArgs a{q, rows, n_qh, kvh, hd, dtype, k_plane, v_plane, n_rows, row_stride,
                     head_stride, block_table, table_cols, table_row_stride, page_size,
                     positions, k_pad, scale, out, ws, ws_bytes};
    int rc = check_rows("kvt_sparse_attend_rows", a);
    if (rc != KVT_OK)
        return rc;
    const int64_t n_ids = block_table ? (int64_t)table_cols * page_size : n_rows;
    const SlotMap sm{block_table, n_ids, n_rows, row_stride, block_table ? page_size : 1,
                     block_table ? table_cols : 0x7fffffff, 0};
    return launch_rows("kvt_sparse_attend_rows", a, k_plane, v_plane, sm, !in_hbm(k_plane, v_plane),
                       stream);
}

// [QSA-KVO] qsa_sparse_attend_rows_staged behind qsa_staging_worthwhile: when the rule holds
// and the staging buffers can take the used pages, the pages are copied into HBM once, in
// logical order, and the rows attend the staged copy; otherwise they read in place.  The
// validity of a position (its page inside the first pages_used, its table entry a page of the
// pool) is the same either way, so both give the same bits.
extern "C" int kvt_sparse_attend_rows_auto(
    const void *q, int32_t rows, int32_t n_qh, int32_t kvh, int32_t hd, int32_t dtype,
    const void *k_plane, const void *v_plane, int64_t n_rows, int64_t row_stride,
    int64_t head_stride, const int32_t *block_table, int32_t pages_used, int32_t page_size,
    const int32_t *positions, int32_t k_pad, float scale, float *out, void *ws, size_t ws_bytes,
    void *staging_k, void *staging_v, size_t staging_bytes, int32_t *staged, void *stream)
{
    const RowsArgs a{q, rows, n_qh, kvh, hd, dtype, k_plane, v_plane, n_rows, row_stride,
                     head_stride, block_table, pages_used, 0, page_size, positions, k_pad,
                     scale, out, ws, ws_bytes};
    if (!block_table || pages_used < 1 || page_size < 1 || n_rows % page_size)
        return kvt::fail(KVT_EINVAL, "kvt_sparse_attend_rows_auto: needs a block table, "
                         "pages_used=%d >= 1 and n_rows=%lld a multiple of page_size=%d",
                         pages_used, (long long)n_rows, page_size);
    int rc = check_rows("kvt_sparse_attend_rows_auto", a);
    if (rc != KVT_OK)
        return rc;
    const int64_t page_bytes = (int64_t)page_size * row_stride;
    const bool fits = staging_k && staging_v && kvt::aligned(staging_k, 16) &&
                      kvt::aligned(staging_v, 16) &&
                      staging_bytes >= (size_t)pages_used * (size_t)page_bytes;
    const bool stage = fits && kvt_staging_worthwhile(rows, k_pad, pages_used, page_size);
    if (staged)
        *staged = stage ? 1 : 0;
    const int64_t n_ids = (int64_t)pages_used * page_size;
    if (!stage) {
        const SlotMap sm{block_table, n_ids, n_rows, row_stride, page_size, pages_used, 0};
        return launch_rows("kvt_sparse_attend_rows_auto", a, k_plane, v_plane, sm,
                           !in_hbm(k_plane, v_plane), stream);
    }
    rc = kvt_stage_pages(k_plane, v_plane, page_bytes, block_table, pages_used,
                         n_rows / page_size, staging_k, staging_v, stream);
    if (rc != KVT_OK)
        return rc;
    const SlotMap sm{block_table, n_ids, n_rows, row_stride, page_size, pages_used, 1};
    return launch_rows("kvt_sparse_attend_rows_auto", a, staging_k, staging_v, sm,
                       !in_hbm(staging_k, staging_v), stream);
}
