// kvt_topk.hip -- S3 index scoring + S4 top-k block selection.
//
// QSA-KVO keeps the pooled indexer plane in HBM because it is scored in full on every step;
// the top-k of those scores decides which K/V blocks cross the host link.
//
// Every score is evaluated in fp64 in index order: each fp16*fp16 product is exact in fp64,
// so the value is fully determined and the selection is reproducible bit for bit.
//
// Wavefront path (k <= 32, the decode case):
//   score_wave_topk -- a workgroup stages 64 pooled rows and the index queries in LDS; lane l
//     of a wave scores row l for one head, so a head's 64 candidates sit one per lane and a
//     64-lane bitonic sort over cross-lane shuffles (no LDS, no barriers) leaves the best k in
//     lanes 0..k-1, written out as a sorted candidate list.
//   merge_wave_topk -- one workgroup per head; each wave folds candidate lists into its running
//     best-32 (the running list in lanes 0..31, the incoming list reversed in lanes 32..63:
//     a bitonic sequence, cleaned in six shuffle steps), then the 16 waves fold pairwise
//     through LDS, and the winners' ids are sorted ascending by one more lane sort.
// Generic path (k up to kMergeMax / 2 = 2048: each merge level at least halves the candidates):
//   score_local_topk -- the same scoring over 128-row chunks, candidates cut to min(k, 128) by
//     a segmented bitonic sort in LDS;  merge_topk -- segments of up to 4096 candidates sorted
//     in LDS and cut to k, repeated until one segment per head remains.
//
// Rank order (a total order, so the result is unique): larger score first, equal scores by
// lower block id, NaN after every number.  Encoded as a 64-bit key (larger = better) plus id.
#include <algorithm>

#include "kvt_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunkBlocks = 128;     // pooled rows per scoring workgroup
constexpr int kMergeThreads = 1024;
constexpr int kMergeMax = 4096;       // candidates per merge workgroup (power of two)
constexpr uint32_t kNoId = 0xffffffffu;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__device__ __forceinline__ uint64_t rank_key(double s)
{
    uint64_t u = __double_as_longlong(s);
    if (s != s)
        return 0;  // NaN: below every number
    if (s == 0.0)
        return 0x8000000000000000ull;  // -0 and +0 are the same score
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// a ranks before b
__device__ __forceinline__ bool better(uint64_t ka, uint32_t ia, uint64_t kb, uint32_t ib)
{
    return ka > kb || (ka == kb && ia < ib);
}

// In-place bitonic sort, best first, of n (power of two) entries split into independent
// segments of `seg` (power of two, seg <= n).  All threads of the block take part.
__device__ void bitonic_best_first(uint64_t *key, uint32_t *id, int n, int seg)
{
    for (int size = 2; size <= seg; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int p = threadIdx.x; p < (n >> 1); p += blockDim.x) {
                // stride is a power of two: i = (p / stride) * 2 * stride + p % stride
                const int i = ((p & ~(stride - 1)) << 1) | (p & (stride - 1));
                const int j = i + stride;
                const bool up = size == seg || (i & size) == 0;
                const uint64_t ka = key[i], kb = key[j];
                const uint32_t ia = id[i], ib = id[j];
                const bool swap = up ? better(kb, ib, ka, ia) : better(ka, ia, kb, ib);
                if (swap) {
                    key[i] = kb; key[j] = ka;
                    id[i] = ib; id[j] = ia;
                }
            }
            __syncthreads();
        }
    }
}

// ascending sort of n (power of two) ids, kNoId last
__device__ void bitonic_ids_ascending(uint32_t *id, int n)
{
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int p = threadIdx.x; p < (n >> 1); p += blockDim.x) {
                const int i = ((p & ~(stride - 1)) << 1) | (p & (stride - 1));
                const int j = i + stride;
                const bool up = size == n || (i & size) == 0;
                const uint32_t a = id[i], b = id[j];
                if (up ? b < a : a < b) {
                    id[i] = b;
                    id[j] = a;
                }
            }
            __syncthreads();
        }
    }
}

__host__ __device__ constexpr int pow2_at_least(int x)
{
    int p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

// grid.x = ceil(n_blocks / kChunkBlocks); dynamic LDS = see score_lds_bytes
__global__ __launch_bounds__(kThreads) void score_local_topk(
    const uint16_t *__restrict__ pooled, int64_t n_blocks, int dim,
    const uint16_t *__restrict__ q_idx, int n_sel, int kk, uint64_t *__restrict__ cand_key,
    uint32_t *__restrict__ cand_id, double *__restrict__ scores_out)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int pitch = dim * 2 + 16;  // bytes per staged pooled row (padded: no bank conflicts)
    unsigned char *rows = lds;
    float *qf = reinterpret_cast<float *>(lds + kChunkBlocks * pitch);
    uint64_t *skey = reinterpret_cast<uint64_t *>(qf + n_sel * dim);
    uint32_t *sid = reinterpret_cast<uint32_t *>(skey + n_sel * kChunkBlocks);

    const int64_t b0 = (int64_t)blockIdx.x * kChunkBlocks;
    const int nrows = (int)std::min<int64_t>(kChunkBlocks, n_blocks - b0);
    const int words_per_row = dim / 8;

    // stage pooled rows (16-byte words, coalesced) and the index queries (as exact fp32)
    for (int w = threadIdx.x; w < nrows * words_per_row; w += kThreads) {
        const int r = w / words_per_row, c = w % words_per_row;
        const uint4 v = *reinterpret_cast<const uint4 *>(pooled + (b0 + r) * dim + c * 8);
        *reinterpret_cast<uint4 *>(rows + r * pitch + c * 16) = v;
    }
    for (int e = threadIdx.x; e < n_sel * dim; e += kThreads)
        qf[e] = f16_bits_to_f32(q_idx[e]);
    __syncthreads();

    // scores: pair p = h*kChunkBlocks + r; four independent fp64 chains per thread
    const int npairs = n_sel * kChunkBlocks;
    for (int p0 = threadIdx.x; p0 < npairs; p0 += 4 * kThreads) {
        int r[4], h[4];
        double acc[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int p = min(p0 + u * kThreads, npairs - 1);
            h[u] = p / kChunkBlocks;
            r[u] = p % kChunkBlocks;
            if (r[u] >= nrows)
                r[u] = 0;
            acc[u] = 0.0;
        }
        for (int c = 0; c < words_per_row; c++) {
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const uint4 v = *reinterpret_cast<const uint4 *>(rows + r[u] * pitch + c * 16);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                const float *qh = qf + h[u] * dim + c * 8;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const uint16_t bits = (uint16_t)(w4[e >> 1] >> ((e & 1) * 16));
                    const double pv = (double)f16_bits_to_f32(bits);
                    acc[u] = fma((double)qh[e], pv, acc[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int p = p0 + u * kThreads;
            if (p >= npairs)
                continue;
            const int hh = p / kChunkBlocks, rr = p % kChunkBlocks;
            if (rr < nrows) {
                skey[p] = rank_key(acc[u]);
                sid[p] = (uint32_t)(b0 + rr);
                if (scores_out)
                    scores_out[(int64_t)hh * n_blocks + b0 + rr] = acc[u];
            } else {
                skey[p] = 0;
                sid[p] = kNoId;
            }
        }
    }
    __syncthreads();

    bitonic_best_first(skey, sid, npairs, kChunkBlocks);

    // best kk of each head's segment -> candidates [h][blockIdx][kk]
    for (int e = threadIdx.x; e < n_sel * kk; e += kThreads) {
        const int hh = e / kk, i = e % kk;
        const int64_t o = ((int64_t)hh * gridDim.x + blockIdx.x) * kk + i;
        cand_key[o] = skey[hh * kChunkBlocks + i];
        cand_id[o] = sid[hh * kChunkBlocks + i];
    }
}

// grid = (n_seg_out, n_sel).  Input per head: n_in candidates; segment s covers
// [s*kMergeMax, ...).  Output per head: n_seg_out*k candidates, or (final) k ids.
__global__ __launch_bounds__(kMergeThreads) void merge_topk(
    const uint64_t *__restrict__ in_key, const uint32_t *__restrict__ in_id, int64_t n_in,
    int k, uint64_t *__restrict__ out_key, uint32_t *__restrict__ out_id,
    int32_t *__restrict__ ids_final)
{
    __shared__ uint64_t skey[kMergeMax];
    __shared__ uint32_t sid[kMergeMax];
    const int h = blockIdx.y;
    const int64_t s0 = (int64_t)blockIdx.x * kMergeMax;
    const int cnt = (int)std::min<int64_t>(kMergeMax, n_in - s0);
    const int n = pow2_at_least(std::max(cnt, k));
    for (int i = threadIdx.x; i < n; i += kMergeThreads) {
        if (i < cnt) {
            skey[i] = in_key[h * n_in + s0 + i];
            sid[i] = in_id[h * n_in + s0 + i];
        } else {
            skey[i] = 0;
            sid[i] = kNoId;
        }
    }
    __syncthreads();
    bitonic_best_first(skey, sid, n, n);
    if (!ids_final) {
        for (int i = threadIdx.x; i < k; i += kMergeThreads) {
            const int64_t o = ((int64_t)h * gridDim.x + blockIdx.x) * k + i;
            out_key[o] = skey[i];
            out_id[o] = sid[i];
        }
        return;
    }
    // final: the k selected ids in ascending order, empty slots (kNoId) last as -1
    const int m = pow2_at_least(k);
    for (int i = threadIdx.x; i < m; i += kMergeThreads)
        if (i >= k)
            sid[i] = kNoId;
    __syncthreads();
    bitonic_ids_ascending(sid, m);
    for (int i = threadIdx.x; i < k; i += kMergeThreads)
        ids_final[h * k + i] = sid[i] == kNoId ? -1 : (int32_t)sid[i];
}


// ---------------------------------------------------------------------------------------------
// wavefront path
// ---------------------------------------------------------------------------------------------
constexpr int kWaveRows = 64;        // pooled rows per scoring workgroup: one per lane
constexpr int kWaveK = 32;           // largest k of this path
constexpr int kMergeWaves = 16;

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src)
{
    const uint32_t lo = __shfl((uint32_t)v, src, 64), hi = __shfl((uint32_t)(v >> 32), src, 64);
    return ((uint64_t)hi << 32) | lo;
}

// The value lane ^ S holds, on the cheapest cross-lane path for S: DPP quad permutes for 1
// and 2, DPP row shifts (up or down by S inside a row of 16) for 4 and 8, a bit-mode
// ds_swizzle for 16, ds_bpermute only for 32.
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane)
{
    const int x = (int)v;
    if constexpr (S == 1)
        return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    else if constexpr (S == 2)
        return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
    else if constexpr (S == 4 || S == 8) {
        const int from_above = __builtin_amdgcn_update_dpp(x, x, 0x100 + S, 0xF, 0xF, false);
        const int from_below = __builtin_amdgcn_update_dpp(x, x, 0x110 + S, 0xF, 0xF, false);
        return (uint32_t)((lane & S) ? from_below : from_above);
    } else if constexpr (S == 16)
        return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x401F);   // and 0x1f, xor 0x10
    else
        return (uint32_t)__shfl_xor(x, S, 64);
}

template <int S>
__device__ __forceinline__ void wave_cx_s(uint64_t &key, uint32_t &id, int lane, bool up)
{
    const uint32_t lo = xor_lane<S>((uint32_t)key, lane);
    const uint32_t hi = xor_lane<S>((uint32_t)(key >> 32), lane);
    const uint32_t pi = xor_lane<S>(id, lane);
    const uint64_t pk = ((uint64_t)hi << 32) | lo;
    const bool lower = (lane & S) == 0;
    const bool mine_better = better(key, id, pk, pi);
    if ((lower == up) != mine_better) {
        key = pk;
        id = pi;
    }
}

// compare-exchange with the lane `stride` away; `up` = this pair ends best-first.  Every call
// site has a compile-time stride once its loop is unrolled, so the switch folds away.
__device__ __forceinline__ void wave_cx(uint64_t &key, uint32_t &id, int lane, int stride, bool up)
{
    switch (stride) {
    case 1: wave_cx_s<1>(key, id, lane, up); break;
    case 2: wave_cx_s<2>(key, id, lane, up); break;
    case 4: wave_cx_s<4>(key, id, lane, up); break;
    case 8: wave_cx_s<8>(key, id, lane, up); break;
    case 16: wave_cx_s<16>(key, id, lane, up); break;
    default: wave_cx_s<32>(key, id, lane, up); break;
    }
}

__device__ __forceinline__ uint32_t xor_lane_dyn(uint32_t v, int lane, int stride)
{
    switch (stride) {
    case 1: return xor_lane<1>(v, lane);
    case 2: return xor_lane<2>(v, lane);
    case 4: return xor_lane<4>(v, lane);
    case 8: return xor_lane<8>(v, lane);
    case 16: return xor_lane<16>(v, lane);
    default: return xor_lane<32>(v, lane);
    }
}

// bitonic sort of the wave's 64 (key, id) pairs, best first
__device__ __forceinline__ void wave_sort_best_first(uint64_t &key, uint32_t &id, int lane)
{
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
            wave_cx(key, id, lane, stride, size == 64 || (lane & size) == 0);
}

// running best-32 (lanes 0..31, best first) merged with a list (lanes 0..31, best first)
__device__ __forceinline__ void wave_merge32(uint64_t &ck, uint32_t &ci, uint64_t lk, uint32_t li,
                                             int lane)
{
    const uint64_t rk = shfl_u64(lk, 63 - lane);
    const uint32_t ri = __shfl(li, 63 - lane, 64);
    if (lane >= 32) {
        ck = rk;
        ci = ri;
    }
#pragma unroll
    for (int stride = 32; stride > 0; stride >>= 1)
        wave_cx(ck, ci, lane, stride, true);
}

// grid.x = ceil(n_blocks / 64), kWaveThreads threads (a wave per head).  LDS: 64 padded rows
// + queries as fp64.
constexpr int kWaveThreads = 512;
__global__ __launch_bounds__(kWaveThreads) void score_wave_topk(
    const uint16_t *__restrict__ pooled, int64_t n_blocks, int dim,
    const uint16_t *__restrict__ q_idx, int n_sel, int k, uint64_t *__restrict__ cand_key,
    uint32_t *__restrict__ cand_id, double *__restrict__ scores_out)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int pitch = dim * 2 + 16;
    unsigned char *rows = lds;
    double *qd = reinterpret_cast<double *>(lds + kWaveRows * pitch);
    const int64_t b0 = (int64_t)blockIdx.x * kWaveRows;
    const int nrows = (int)std::min<int64_t>(kWaveRows, n_blocks - b0);
    const int wpr = dim / 8;

    // every load is issued unconditionally (tail rows re-read the last valid row)
    constexpr int kMaxWordsPerThread = kWaveRows * (256 / 8) / kWaveThreads;   // 4
    u32x4 v[kMaxWordsPerThread];
#pragma unroll
    for (int u = 0; u < kMaxWordsPerThread; u++) {
        const int w = threadIdx.x + u * kWaveThreads;
        const int r = min(w / wpr, nrows - 1), c = w % wpr;
        if (w < kWaveRows * wpr)
            v[u] = *reinterpret_cast<const u32x4 *>(pooled + (b0 + r) * dim + c * 8);
    }
#pragma unroll
    for (int u = 0; u < kMaxWordsPerThread; u++) {
        const int w = threadIdx.x + u * kWaveThreads;
        if (w < kWaveRows * wpr)
            *reinterpret_cast<u32x4 *>(rows + (w / wpr) * pitch + (w % wpr) * 16) = v[u];
    }
    for (int e = threadIdx.x; e < n_sel * dim; e += kWaveThreads)
        qd[e] = (double)f16_bits_to_f32(q_idx[e]);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool valid = lane < nrows;
    const unsigned char *my_row = rows + lane * pitch;
    // one head per wave: lane l scores row l, one fp64 chain in index order
    for (int h = wave; h < n_sel; h += kWaveThreads / 64) {
        const double *qh = qd + h * dim;
        double acc = 0.0;
        for (int c = 0; c < wpr; c++) {
            const u32x4 w4 = *reinterpret_cast<const u32x4 *>(my_row + c * 16);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint16_t bits = (uint16_t)(w4[e >> 1] >> ((e & 1) * 16));
                acc = fma(qh[c * 8 + e], (double)f16_bits_to_f32(bits), acc);
            }
        }
        uint64_t key = valid ? rank_key(acc) : 0;
        uint32_t id = valid ? (uint32_t)(b0 + lane) : kNoId;
        if (scores_out && valid)
            scores_out[(int64_t)h * n_blocks + b0 + lane] = acc;
        wave_sort_best_first(key, id, lane);
        if (lane < k) {
            const int64_t o = ((int64_t)h * gridDim.x + blockIdx.x) * k + lane;
            cand_key[o] = key;
            cand_id[o] = id;
        }
    }
}

// grid.x = n_sel, kMergeWaves*64 threads.  Lists of k sorted candidates: [h][n_lists][k].
__global__ __launch_bounds__(kMergeWaves * 64) void merge_wave_topk(
    const uint64_t *__restrict__ cand_key, const uint32_t *__restrict__ cand_id, int n_lists,
    int k, int32_t *__restrict__ ids)
{
    __shared__ uint64_t skey[kMergeWaves][kWaveK];
    __shared__ uint32_t sid[kMergeWaves][kWaveK];
    const int h = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t *hk = cand_key + (int64_t)h * n_lists * k;
    const uint32_t *hi = cand_id + (int64_t)h * n_lists * k;
    const int li = min(lane, k - 1);
    uint64_t ck = 0;
    uint32_t ci = kNoId;
    // prefetch one list ahead: the loads of list L+16 are in flight while L merges
    int L = wave;
    uint64_t nk = 0;
    uint32_t ni = kNoId;
    if (L < n_lists) {
        nk = hk[(int64_t)L * k + li];
        ni = hi[(int64_t)L * k + li];
    }
    while (L < n_lists) {
        uint64_t lk = lane < k ? nk : 0;
        uint32_t lid = lane < k ? ni : kNoId;
        const int Ln = L + kMergeWaves;
        if (Ln < n_lists) {
            nk = hk[(int64_t)Ln * k + li];
            ni = hi[(int64_t)Ln * k + li];
        }
        wave_merge32(ck, ci, lk, lid, lane);
        L = Ln;
    }
    // pairwise fold of the waves' lists through LDS
    for (int active = kMergeWaves / 2; active >= 1; active >>= 1) {
        if (wave >= active && wave < 2 * active && lane < kWaveK) {
            skey[wave][lane] = ck;
            sid[wave][lane] = ci;
        }
        __syncthreads();
        if (wave < active) {
            const uint64_t lk = skey[wave + active][lane & 31];
            const uint32_t lid = sid[wave + active][lane & 31];
            wave_merge32(ck, ci, lane < kWaveK ? lk : 0, lane < kWaveK ? lid : kNoId, lane);
        }
        __syncthreads();
    }
    if (wave == 0) {
        // the k winners' ids in ascending order; empty slots (kNoId) sort last and become -1
        uint32_t id = lane < k ? ci : kNoId;
#pragma unroll
        for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const uint32_t p = xor_lane_dyn(id, lane, stride);
                const bool lower = (lane & stride) == 0;
                const bool up = size == 64 || (lane & size) == 0;
                const bool mine_first = id < p;
                if ((lower == up) != mine_first && id != p)
                    id = p;
            }
        if (lane < k)
            ids[h * k + lane] = id == kNoId ? -1 : (int32_t)id;
    }
}

size_t score_lds_bytes(int dim, int n_sel)
{
    return (size_t)kChunkBlocks * (dim * 2 + 16) + (size_t)n_sel * dim * 4 +
           (size_t)n_sel * kChunkBlocks * 12;
}

struct Plan {
    int64_t n_wg;        // scoring workgroups
    int kk;              // candidates each keeps per head
    int64_t level0;      // candidates per head after scoring
    int64_t buf_a, buf_b;  // entries per head of the two ping-pong candidate buffers
};

Plan make_plan(int64_t n_blocks, int k)
{
    Plan p;
    p.n_wg = (n_blocks + kChunkBlocks - 1) / kChunkBlocks;
    p.kk = std::min(k, kChunkBlocks);
    p.level0 = p.n_wg * p.kk;
    p.buf_a = p.level0;
    int64_t n = p.level0, b = 0;
    bool to_b = true;
    while (n > kMergeMax) {  // intermediate merge levels
        const int64_t segs = (n + kMergeMax - 1) / kMergeMax;
        n = segs * k;
        if (to_b)
            b = std::max(b, n);
        to_b = !to_b;
    }
    p.buf_b = b;
    return p;
}

}  // namespace

extern "C" size_t kvt_index_topk_ws_bytes(int64_t n_blocks, int32_t n_sel, int32_t k)
{
    if (n_blocks < 0 || n_sel < 1 || k < 1)
        return 0;
    if (k <= kWaveK) {
        const size_t c = (size_t)n_sel * (size_t)std::max<int64_t>((n_blocks + kWaveRows - 1) / kWaveRows, 1) * k;
        return round_up(c * 8, 256) + round_up(c * 4, 256) + 256;
    }
    const Plan p = make_plan(std::max<int64_t>(n_blocks, 1), k);
    const size_t a = (size_t)n_sel * p.buf_a, b = (size_t)n_sel * p.buf_b;
    return round_up(a * 8, 256) + round_up(a * 4, 256) + round_up(b * 8, 256) +
           round_up(b * 4, 256) + 256;
}

// S3+S4: QSA-KVO pooled-plane scoring and top-k block selection.
extern "C" int kvt_index_topk(const void *pooled, int64_t n_blocks, int32_t dim,
                              const void *q_idx, int32_t n_sel, int32_t k, int32_t *ids,
                              double *scores, void *ws, size_t ws_bytes, void *stream)
{
    if (n_blocks < 0 || n_blocks > 0x7fffffffll || dim < 8 || dim > 256 || dim % 8 ||
        n_sel < 1 || n_sel > 32 || k < 1 || k > kMergeMax / 2)
        return kvt::fail(KVT_EINVAL,
                         "kvt_index_topk: n_blocks=%lld dim=%d n_sel=%d k=%d outside limits",
                         (long long)n_blocks, dim, n_sel, k);
    if (!ids || !q_idx || (n_blocks && !pooled))
        return kvt::fail(KVT_EINVAL, "kvt_index_topk: null pointer");
    if (!kvt::aligned(pooled, 16))
        return kvt::fail(KVT_EALIGN, "kvt_index_topk: pooled plane must be 16-byte aligned");
    const size_t need = kvt_index_topk_ws_bytes(n_blocks, n_sel, k);
    if (!ws || ws_bytes < need)
        return kvt::fail(KVT_EINVAL, "kvt_index_topk: workspace of %zu bytes, need %zu",
                         ws_bytes, need);
    hipStream_t s = kvt::as_stream(stream);
    if (k <= kWaveK) {
        const int64_t n_wg = (n_blocks + kWaveRows - 1) / kWaveRows;
        const size_t c = (size_t)n_sel * (size_t)std::max<int64_t>(n_wg, 1) * k;
        uintptr_t w = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
        uint64_t *ck = reinterpret_cast<uint64_t *>(w);
        uint32_t *ci = reinterpret_cast<uint32_t *>(w + round_up(c * 8, 256));
        if (n_wg > 0) {
            const size_t lds = (size_t)kWaveRows * (dim * 2 + 16) + (size_t)n_sel * dim * 8;
            hipLaunchKernelGGL(score_wave_topk, dim3((unsigned)n_wg), dim3(kWaveThreads), lds, s,
                               static_cast<const uint16_t *>(pooled), n_blocks, dim,
                               static_cast<const uint16_t *>(q_idx), n_sel, k, ck, ci, scores);
            KVT_LAUNCHED("score_wave_topk");
        }
        hipLaunchKernelGGL(merge_wave_topk, dim3(n_sel), dim3(kMergeWaves * 64), 0, s, ck, ci,
                           (int)n_wg, k, ids);
        KVT_LAUNCHED("merge_wave_topk");
        return KVT_OK;
    }
    const Plan p = make_plan(std::max<int64_t>(n_blocks, 1), k);

    // carve the workspace (256-byte aligned pieces)
    uintptr_t w = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
    const size_t a = (size_t)n_sel * p.buf_a, b = (size_t)n_sel * p.buf_b;
    uint64_t *a_key = reinterpret_cast<uint64_t *>(w); w += round_up(a * 8, 256);
    uint32_t *a_id = reinterpret_cast<uint32_t *>(w); w += round_up(a * 4, 256);
    uint64_t *b_key = reinterpret_cast<uint64_t *>(w); w += round_up(b * 8, 256);
    uint32_t *b_id = reinterpret_cast<uint32_t *>(w);

    if (n_blocks == 0) {
        // nothing to rank: every slot is empty.  One merge over a single empty segment.
        hipLaunchKernelGGL(merge_topk, dim3(1, n_sel), dim3(kMergeThreads), 0, s, a_key, a_id,
                           (int64_t)0, k, nullptr, nullptr, ids);
        KVT_LAUNCHED("merge_topk");
        return KVT_OK;
    }
    const size_t lds = score_lds_bytes(dim, n_sel);
    if (lds > 160 * 1024)
        return kvt::fail(KVT_EINVAL, "kvt_index_topk: dim=%d n_sel=%d need %zu bytes of LDS",
                         dim, n_sel, lds);
    hipLaunchKernelGGL(score_local_topk, dim3((unsigned)p.n_wg), dim3(kThreads), lds, s,
                       static_cast<const uint16_t *>(pooled), n_blocks, dim,
                       static_cast<const uint16_t *>(q_idx), n_sel, p.kk, a_key, a_id, scores);
    KVT_LAUNCHED("score_local_topk");

    int64_t n = p.level0;
    bool in_a = true;
    while (true) {
        const int64_t segs = (n + kMergeMax - 1) / kMergeMax;
        const uint64_t *ik = in_a ? a_key : b_key;
        const uint32_t *ii = in_a ? a_id : b_id;
        if (segs == 1) {
            hipLaunchKernelGGL(merge_topk, dim3(1, n_sel), dim3(kMergeThreads), 0, s, ik, ii, n,
                               k, nullptr, nullptr, ids);
            KVT_LAUNCHED("merge_topk");
            return KVT_OK;
        }
        uint64_t *ok = in_a ? b_key : a_key;
        uint32_t *oi = in_a ? b_id : a_id;
        hipLaunchKernelGGL(merge_topk, dim3((unsigned)segs, n_sel), dim3(kMergeThreads), 0, s,
                           ik, ii, n, k, ok, oi, nullptr);
        KVT_LAUNCHED("merge_topk");
        n = segs * k;
        in_a = !in_a;
    }
}

namespace {

// grid = n_sel, 256 threads.  ids[h] ascending, -1 only at the end (kvt_index_topk's output).
__global__ __launch_bounds__(256) void select_positions_kernel(const int32_t *__restrict__ ids,
                                                               int k, int cr, int64_t n_tok,
                                                               int k_pad,
                                                               int32_t *__restrict__ positions)
{
    const int h = blockIdx.x;
    const int32_t *hid = ids + (int64_t)h * k;
    // valid ids form a prefix: find its length by bisection on "id >= 0"
    int lo = 0, hi = k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (hid[mid] >= 0)
            lo = mid + 1;
        else
            hi = mid;
    }
    const int64_t n_sel_tok = (int64_t)lo * cr;
    const int64_t tail0 = n_tok / cr * cr;           // first token not in a complete block
    const int64_t n_tail = n_tok - tail0;
    int32_t *out = positions + (int64_t)h * k_pad;
    for (int j = threadIdx.x; j < k_pad; j += 256) {
        int64_t p = -1;
        if (j < n_sel_tok)
            p = (int64_t)hid[j / cr] * cr + j % cr;
        else if (j - n_sel_tok < n_tail)
            p = tail0 + (j - n_sel_tok);
        out[j] = (int32_t)p;
    }
}

}  // namespace

// QSA-KVO selection geometry: the indexer selects pooled blocks of cr tokens; a row attends their
// positions plus the write head's tail (the < cr newest tokens no complete block covers),
// padded with -1 to K_pad = ceil((block_topk*cr + cr - 1) / 32) * 32.
extern "C" int kvt_select_positions(const int32_t *ids, int32_t n_sel, int32_t k, int32_t cr,
                                    int64_t n_tok, int32_t k_pad, int32_t *positions,
                                    void *stream)
{
    if (n_sel < 1 || k < 1 || cr < 1 || n_tok < 0 || n_tok > 0x7fffffffll ||
        (int64_t)k * cr + cr - 1 > k_pad)
        return kvt::fail(KVT_EINVAL,
                         "kvt_select_positions: n_sel=%d k=%d cr=%d n_tok=%lld k_pad=%d (need "
                         "k_pad >= k*cr + cr - 1)",
                         n_sel, k, cr, (long long)n_tok, k_pad);
    if (!ids || !positions)
        return kvt::fail(KVT_EINVAL, "kvt_select_positions: null pointer");
    hipLaunchKernelGGL(select_positions_kernel, dim3(n_sel), dim3(256), 0, kvt::as_stream(stream),
                       ids, k, cr, n_tok, k_pad, positions);
    KVT_LAUNCHED("select_positions_kernel");
    return KVT_OK;
}
