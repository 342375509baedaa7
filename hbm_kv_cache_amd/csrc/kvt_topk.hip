// kvt_topk.hip -- S3 index scoring + S4 top-k block selection.
//
// QSA-KVO keeps the pooled indexer plane in HBM because it is scored in full on every step;
// the top-k of those scores decides which K/V blocks cross the host link.
//
// Every score is evaluated in fp64 in index order: each fp16*fp16 product is exact in fp64,
// so the value is fully determined and the selection is reproducible bit for bit.
//
// Wavefront path (k <= 32, the decode case):
//   score_wave_topk -- a workgroup stages 128 pooled rows and two heads' index queries in LDS;
//     lane l of a wave scores one row for one head, so 64 of a head's candidates sit one per
//     lane and a 64-lane bitonic sort over cross-lane shuffles (no barriers) leaves the best 32
//     in lanes 0..31; the head's two waves merge their lists in LDS and write the best k as a
//     sorted candidate list.
//   merge_wave_topk -- one workgroup per head; each half-wave folds candidate lists into its
//     running best-32 (each incoming list read in reverse order, so the better entry of every
//     lane pair is a bitonic sequence, cleaned in five shuffle steps), then the halves and the
//     8 or 16 waves fold pairwise, and the winners' ids are sorted ascending by one more lane sort.
// Selection path (32 < k <= 2048):
//   score_wave_topk<true> -- the same scoring (64 rows, eight heads per workgroup), writing
//     every rank key;  select_level -- exact
//     selection by bisection over the (key, id) composite, per segment of up to 4096 keys (8192
//     for k >= 1024), then once more over the survivors (up to 8192), whose output is already in
//     id order.
//
// Rank order (a total order, so the result is unique): larger score first, equal scores by
// lower block id, NaN after every number.  Encoded as a 64-bit key (larger = better) plus id.
#include <algorithm>

#include "kvt_internal.h"

namespace {

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

// ---------------------------------------------------------------------------------------------
// wavefront path
// ---------------------------------------------------------------------------------------------
constexpr int kWaveRows = 64;        // pooled rows per scoring workgroup: one per lane
constexpr int kWaveK = 32;           // largest k of this path

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

// Each 32-lane half of a wave merges on its own: a running best-32 (slot = lane & 31, best
// first) and a list held reversed (slot 31 - (lane & 31) of a best-first list).  The better of
// the two in every lane is the best 32 of both, as a bitonic sequence (falling, then rising),
// which five compare-exchange steps inside the half sort best first.  A list is reversed by
// the address its lanes read, so a merge costs one compare and five steps on half a wave.
__device__ __forceinline__ void half_merge32(uint64_t &ck, uint32_t &ci, uint64_t rk, uint32_t ri,
                                             int lane)
{
    if (better(rk, ri, ck, ci)) {
        ck = rk;
        ci = ri;
    }
#pragma unroll
    for (int stride = 16; stride > 0; stride >>= 1)
        wave_cx(ck, ci, lane, stride, true);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// The exact product of two fp16 values in fp32 (11-bit significands give at most 22 bits, and
// the exponents stay inside fp32's normal range), as one v_fma_mix_f32 that adds `zero`.  The
// zero is 0.0f passed in from the host, so the compiler keeps the mixed-precision FMA instead
// of converting both operands first.  Adding it to the fp64 sum is then exactly the fp64 FMA
// of the two values.
__device__ __forceinline__ float f16_product(_Float16 a, _Float16 b, float zero)
{
    return __builtin_fmaf((float)a, (float)b, zero);
}

// Scoring workgroup shapes.  The list path (k <= 32) takes 128 pooled rows and two heads, two
// waves per head (rows 0..63 and 64..127), four waves in all: the scoring chains and sorts
// spread over many CUs at one wave per SIMD (the loop is VALU-bound), and the two waves of a
// head merge their best-32 lists in LDS, so the merge kernel reads one list per 128 rows.  The
// keys-only path (the selection path's input) has no lists to merge: 64 rows and eight heads,
// a wave per head, so each staged row serves eight chains.
template <bool kKeysOnly>
struct ScoreShape {
    static constexpr int kParts = kKeysOnly ? 1 : 2;       // waves per head, 64 rows each
    static constexpr int kHeads = kKeysOnly ? 8 : 2;       // heads per workgroup
    static constexpr int kRows = kParts * kWaveRows;
    static constexpr int kThreads = kHeads * kParts * 64;
    // 16-byte words of the row and the query held in registers per batch of the scoring chain:
    // the list path runs one workgroup per CU at a time and takes 128 elements a batch; the
    // keys-only path runs many workgroups per CU and keeps to fewer registers
    static constexpr int kBatch = kKeysOnly ? 8 : 16;
    static size_t lds_bytes(int dim)
    {
        return (size_t)kRows * (dim * 2 + 16) + (size_t)kHeads * dim * 2 +
               (kKeysOnly ? 0 : (size_t)kHeads * kWaveK * 12);
    }
};
constexpr int kScoreRows = ScoreShape<false>::kRows;   // rows per candidate list
// grid.x = n_rg * ceil(n_sel / kHeads) with n_rg = ceil(n_blocks / kRows): row group
// blockIdx.x % n_rg, head group blockIdx.x / n_rg.  Workgroups go to the eight XCDs in turn, so
// with n_rg a multiple of 8 every head group of a row group runs on one XCD and its rows come
// from HBM once.  LDS: the padded rows, the group's index queries (fp16), the upper waves' lists.
// kKeysOnly: write every row's rank key to cand_key[h][n_blocks] (ids implicit) instead of the
// sorted best-k candidate lists [h][n_rg][k] -- the input of the selection path.
template <bool kKeysOnly>
__global__ __launch_bounds__(ScoreShape<kKeysOnly>::kThreads) void score_wave_topk(
    const uint16_t *__restrict__ pooled, int64_t n_blocks, int dim,
    const uint16_t *__restrict__ q_idx, int n_sel, int k, uint64_t *__restrict__ cand_key,
    uint32_t *__restrict__ cand_id, double *__restrict__ scores_out, float zero)
{
    using Sh = ScoreShape<kKeysOnly>;
    constexpr int kRows = Sh::kRows, kHeads = Sh::kHeads, kParts = Sh::kParts;
    constexpr int kThreads = Sh::kThreads;
    extern __shared__ __align__(16) unsigned char lds[];
    const int pitch = dim * 2 + 16;
    unsigned char *rows = lds;
    uint16_t *qs = reinterpret_cast<uint16_t *>(lds + kRows * pitch);
    uint64_t *list_key = reinterpret_cast<uint64_t *>(lds + kRows * pitch + kHeads * dim * 2);
    uint32_t *list_id = reinterpret_cast<uint32_t *>(list_key + kHeads * kWaveK);
    const unsigned n_rg = (unsigned)((n_blocks + kRows - 1) / kRows);
    const unsigned rg = blockIdx.x % n_rg;
    const int h0 = (int)(blockIdx.x / n_rg) * kHeads;
    const int64_t b0 = (int64_t)rg * kRows;
    const int nrows = (int)std::min<int64_t>(kRows, n_blocks - b0);
    const int wpr = dim / 8;

    // every load is issued unconditionally (tail rows re-read the last valid row)
    constexpr int kMaxWordsPerThread = kRows * (256 / 8) / kThreads;   // 16 or 4
    u32x4 v[kMaxWordsPerThread];
#pragma unroll
    for (int u = 0; u < kMaxWordsPerThread; u++) {
        const int w = threadIdx.x + u * kThreads;
        const int r = min(w / wpr, nrows - 1), c = w % wpr;
        if (w < kRows * wpr)
            v[u] = *reinterpret_cast<const u32x4 *>(pooled + (b0 + r) * dim + c * 8);
    }
#pragma unroll
    for (int u = 0; u < kMaxWordsPerThread; u++) {
        const int w = threadIdx.x + u * kThreads;
        if (w < kRows * wpr)
            *reinterpret_cast<u32x4 *>(rows + (w / wpr) * pitch + (w % wpr) * 16) = v[u];
    }
    const int nh = std::min(kHeads, n_sel - h0);
    for (int e = threadIdx.x; e < nh * dim; e += kThreads)
        qs[e] = q_idx[h0 * dim + e];
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hl = wave / kParts, part = wave % kParts;   // head in the group, row half
    const int row = part * kWaveRows + lane;
    const bool valid = row < nrows;
    const unsigned char *my_row = rows + row * pitch;
    uint64_t key = 0;
    uint32_t id = kNoId;
    // lane l of a wave scores its row for one head, one fp64 chain in index order.  kBatch words
    // (8 elements each) of the row and the query are read into registers at once, so the chain
    // waits on LDS once per batch.
    if (hl < nh) {
        const int h = h0 + hl;
        const unsigned char *q_row = reinterpret_cast<const unsigned char *>(qs + hl * dim);
        double acc = 0.0;
        constexpr int kBatch = Sh::kBatch;
        for (int c0 = 0; c0 < wpr; c0 += kBatch) {
            u32x4 kw[kBatch], qw[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; j++) {   // words past the row re-read its last word, unused
                const int c = min(c0 + j, wpr - 1);
                kw[j] = *reinterpret_cast<const u32x4 *>(my_row + c * 16);
                qw[j] = *reinterpret_cast<const u32x4 *>(q_row + c * 16);
            }
#pragma unroll
            for (int j = 0; j < kBatch; j++)
                if (c0 + j < wpr)
#pragma unroll
                    for (int e = 0; e < 4; e++) {   // word e: elements 2e (low half), 2e + 1
                        // (the words are copied out first: clang's bit_cast of a vector
                        // element subscript reads element 0 whatever the index)
                        const uint32_t kv = kw[j][e], qv = qw[j][e];
                        const half2_t kx = __builtin_bit_cast(half2_t, kv);
                        const half2_t qx = __builtin_bit_cast(half2_t, qv);
                        acc += (double)f16_product(qx[0], kx[0], zero);
                        acc += (double)f16_product(qx[1], kx[1], zero);
                    }
        }
        key = valid ? rank_key(acc) : 0;
        id = valid ? (uint32_t)(b0 + row) : kNoId;
        if (scores_out && valid)
            scores_out[(int64_t)h * n_blocks + b0 + row] = acc;
        if (kKeysOnly) {
            if (valid)
                cand_key[(int64_t)h * n_blocks + b0 + row] = key;
        } else {
            wave_sort_best_first(key, id, lane);
            if (part == 1 && lane < kWaveK) {
                list_key[hl * kWaveK + lane] = key;
                list_id[hl * kWaveK + lane] = id;
            }
        }
    }
    if constexpr (!kKeysOnly) {
        __syncthreads();
        // the lower wave takes the upper wave's best 32, read in reverse order
        if (hl < nh && part == 0) {
            const int sl = kWaveK - 1 - (lane & 31);
            half_merge32(key, id, list_key[hl * kWaveK + sl], list_id[hl * kWaveK + sl], lane);
            if (lane < k) {
                const int64_t o = ((int64_t)(h0 + hl) * n_rg + rg) * k + lane;
                cand_key[o] = key;
                cand_id[o] = id;
            }
        }
    }
}

// grid.x = n_sel, kMergeWaves*64 threads.  Lists of k sorted candidates: [h][n_lists][k].
// Half-wave hw (2 * wave + upper half) keeps a running best-32 over lists hw, hw + 2W, ...;
// then the upper half of each wave folds into the lower, and the waves fold pairwise through
// LDS.  Slots past a list's k entries, and lists past n_lists, are empty (key 0, id kNoId):
// merging an empty list leaves a sorted list as it is.  A fold level costs about two merge
// rounds, so few lists take 8 waves and many take 16.
template <int kMergeWaves>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_wave_topk(
    const uint64_t *__restrict__ cand_key, const uint32_t *__restrict__ cand_id, int n_lists,
    int k, int32_t *__restrict__ ids)
{
    constexpr int kHalves = 2 * kMergeWaves;
    __shared__ uint64_t skey[kMergeWaves][kWaveK];
    __shared__ uint32_t sid[kMergeWaves][kWaveK];
    const int h = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane & 31, hw = 2 * wave + (lane >> 5);
    const uint64_t *hk = cand_key + (int64_t)h * n_lists * k;
    const uint32_t *hi = cand_id + (int64_t)h * n_lists * k;
    auto load = [&](int L, int sl, uint64_t &key, uint32_t &id) {
        const bool in = L < n_lists && sl < k;
        key = in ? hk[(int64_t)L * k + sl] : 0;
        id = in ? hi[(int64_t)L * k + sl] : kNoId;
    };
    uint64_t ck, nk;
    uint32_t ci, ni;
    load(hw, slot, ck, ci);
    // one list ahead: the loads of round r + 1 are in flight while round r merges
    const int rounds = (n_lists + kHalves - 1) / kHalves;
    load(hw + kHalves, 31 - slot, nk, ni);
    for (int r = 1; r < rounds; r++) {
        const uint64_t lk = nk;
        const uint32_t lid = ni;
        load(hw + (r + 1) * kHalves, 31 - slot, nk, ni);
        half_merge32(ck, ci, lk, lid, lane);
    }
    // the upper half's list, reversed, into the lower half (lane l < 32 reads lane 63 - l)
    {
        const uint64_t rk = shfl_u64(ck, 63 - lane);
        const uint32_t ri = __shfl(ci, 63 - lane, 64);
        half_merge32(ck, ci, rk, ri, lane);
    }
    // pairwise fold of the waves' lists (lanes 0..31) through LDS, read back reversed.  A wave
    // writes its slot once, at the level where it hands its list on, so one barrier a level
    // orders every write before its read.
#pragma unroll
    for (int active = kMergeWaves / 2; active >= 1; active >>= 1) {
        if (wave >= active && wave < 2 * active && lane < kWaveK) {
            skey[wave][lane] = ck;
            sid[wave][lane] = ci;
        }
        __syncthreads();
        if (wave < active)
            half_merge32(ck, ci, skey[wave + active][31 - slot], sid[wave + active][31 - slot], lane);
    }
    if (wave == 0) {
        // the k winners' ids in ascending order (a sort inside each half; the lower half's is
        // used); empty slots (kNoId) sort last and become -1
        uint32_t id = lane < k ? ci : kNoId;
#pragma unroll
        for (int size = 2; size <= 32; size <<= 1)
#pragma unroll
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const uint32_t p = xor_lane_dyn(id, lane, stride);
                const bool lower = (lane & stride) == 0;
                const bool up = size == 32 || (lane & size) == 0;
                const bool mine_first = id < p;
                if ((lower == up) != mine_first && id != p)
                    id = p;
            }
        if (lane < k)
            ids[h * k + lane] = id == kNoId ? -1 : (int32_t)id;
    }
}

// ---------------------------------------------------------------------------------------------
// selection path (32 < k <= 2048)
// ---------------------------------------------------------------------------------------------
// Every element is ranked by the composite (rank key, ~id): 96 bits, larger = better, unique, so
// the top k are exactly the elements at or above the k-th largest composite T.  A workgroup
// holds one segment of a head's list in registers (element i = e*1024 + thread), finds T a
// byte at a time from 256-bin LDS histograms -- two barriers a pass, starting at the first byte
// in which the keys differ, stopping once a bin holds exactly the elements still needed -- and
// writes the elements >= T in element order.  Level 0 reads the rank keys of the scoring pass (ids =
// positions, ascending); every level keeps its output in id order, so the last level's output
// is the answer already sorted by id.  Empty slots (key 0, id kNoId) rank below every element.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelFinalE = 8;                       // the last level: up to 8192 candidates
// Elements per thread of an intermediate level: segments of 4096, or of 8192 for k >= 1024,
// where a 4096-element segment would keep a quarter or more of its elements and the levels
// would shrink slowly (top-2048 of 65,535: 53 against 62 us).
inline int sel_seg_e(int k) { return k >= 1024 ? 8 : 4; }

// the workgroup's sum of one count per wave (one barrier; red is used by this call only)
__device__ __forceinline__ int block_sum(int c, int *red, int wave, int lane)
{
    if (lane == 0)
        red[wave] = c;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; w++)
        tot += red[w];
    return __builtin_amdgcn_readfirstlane(tot);
}

// grid = (segments, n_sel).  in_id NULL: ids are the element positions.  Output: per segment
// k slots (the selected elements in order, then empty slots), or with ids_final the head's k
// ids, -1 for empty slots.
template <int E>
__global__ __launch_bounds__(kSelThreads) void select_level(
    const uint64_t *__restrict__ in_key, const uint32_t *__restrict__ in_id, int64_t n_in, int k,
    uint64_t *__restrict__ out_key, uint32_t *__restrict__ out_id, int32_t *__restrict__ ids_final)
{
    constexpr int kSlots = E * kSelWaves;   // (element slab, wave) counts, <= 128
    __shared__ int red[kSelWaves];
    __shared__ int off[kSlots + 1];
    __shared__ int hist[256];
    __shared__ int pick[3];
    __shared__ uint64_t rmin[kSelWaves], rmax[kSelWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y;
    const int64_t s0 = (int64_t)blockIdx.x * (E * kSelThreads);
    const uint64_t *hk = in_key + (int64_t)h * n_in;
    const uint32_t *hi = in_id ? in_id + (int64_t)h * n_in : nullptr;
    uint64_t key[E];
    uint32_t lo[E];
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int64_t i = s0 + e * kSelThreads + tid;
        const bool in = i < n_in;
        const int64_t ic = in ? i : 0;
        const uint64_t kv = hk[ic];
        const uint32_t id = hi ? hi[ic] : (uint32_t)ic;
        key[e] = in ? kv : 0;
        lo[e] = in ? ~id : 0;     // an empty slot (id kNoId) also ranks 0
    }
    // T = the largest composite with count(>= T) >= k; stays 0 with k or fewer elements.
    // Radix search, 8 bits a pass: a 256-bin LDS histogram of the next byte over the elements
    // that still match the bytes chosen so far, then the bin holding the k-th largest.  The
    // 64 key bits first; the 32 id bits only when the k-th and (k+1)-th keys are equal.  A
    // pass ends the search when its bin holds exactly the elements still needed.
    uint64_t tk = 0;
    uint32_t tl = 0;
    bool valid[E];
    int nv = 0;
#pragma unroll
    for (int e = 0; e < E; e++) {
        valid[e] = (key[e] | lo[e]) != 0;
        nv += __popcll(__ballot(valid[e]));
    }
    nv = block_sum(nv, red, wave, lane);
    if (nv > k) {
        // Leading key bytes that every valid element shares (those of the smallest and the
        // largest key) would each take a pass that puts all elements in one bin: T starts with
        // them, and the search at the first byte where the keys differ.  Candidate lists (the
        // levels after the first) hold the top of each head's scores, which share leading
        // bytes; the first level's raw scores span both signs, so it goes straight to pass 0.
        int common = 0;
        if (hi) {
            uint64_t kmin = ~0ull, kmax = 0;
#pragma unroll
            for (int e = 0; e < E; e++)
                if (valid[e]) {
                    kmin = key[e] < kmin ? key[e] : kmin;
                    kmax = key[e] > kmax ? key[e] : kmax;
                }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const uint64_t a = shfl_u64(kmin, lane ^ d), b = shfl_u64(kmax, lane ^ d);
                kmin = a < kmin ? a : kmin;
                kmax = b > kmax ? b : kmax;
            }
            if (lane == 0) {
                rmin[wave] = kmin;
                rmax[wave] = kmax;
            }
            __syncthreads();
#pragma unroll
            for (int w = 0; w < kSelWaves; w++) {
                kmin = rmin[w] < kmin ? rmin[w] : kmin;
                kmax = rmax[w] > kmax ? rmax[w] : kmax;
            }
            common = kmin == kmax ? 8 : __builtin_clzll(kmin ^ kmax) >> 3;
            tk = common == 0 ? 0 : common == 8 ? kmin : kmin >> (64 - 8 * common) << (64 - 8 * common);
        }
        int need = k;          // elements still to take from the matching ones
        bool done = false;
        for (int pass = common; pass < 12 && !done; pass++) {   // 8 key bytes, then 4 id bytes
            const bool on_key = pass < 8;
            const int shift = on_key ? 56 - 8 * pass : 24 - 8 * (pass - 8);
            for (int b = tid; b < 256; b += kSelThreads)
                hist[b] = 0;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < E; e++) {
                bool match;
                uint32_t digit;
                if (on_key) {
                    match = valid[e] && (shift == 56 || (key[e] >> (shift + 8)) == (tk >> (shift + 8)));
                    digit = (uint32_t)(key[e] >> shift) & 255u;
                } else {
                    match = valid[e] && key[e] == tk &&
                            (shift == 24 || (lo[e] >> (shift + 8)) == (tl >> (shift + 8)));
                    digit = (lo[e] >> shift) & 255u;
                }
                if (match)
                    atomicAdd(&hist[digit], 1);
            }
            __syncthreads();
            // wave 0: bins from the top, the digit whose bin reaches `need`
            if (wave == 0) {
                int c[4], loc = 0;
#pragma unroll
                for (int j = 0; j < 4; j++) {   // lane L holds bins 255-4L .. 252-4L
                    c[j] = hist[255 - 4 * lane - j];
                    loc += c[j];
                }
                int incl = loc;                  // inclusive prefix over lanes (from the top)
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int t = __shfl_up(incl, d, 64);
                    if (lane >= d)
                        incl += t;
                }
                int before = incl - loc;         // elements in higher bins than this lane's
                int dig = -1, above = 0, inbin = 0;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    if (dig < 0 && before + c[j] >= need) {
                        dig = 255 - 4 * lane - j;
                        above = before;
                        inbin = c[j];
                    }
                    before += c[j];
                }
                const uint64_t hit = __ballot(dig >= 0);
                const int src = (int)__builtin_ctzll(hit);   // the first lane from the top
                dig = __shfl(dig, src, 64);
                above = __shfl(above, src, 64);
                inbin = __shfl(inbin, src, 64);
                if (lane == 0) {
                    pick[0] = dig;
                    pick[1] = above;
                    pick[2] = inbin;
                }
            }
            __syncthreads();
            const int dig = pick[0];
            need -= pick[1];
            if (on_key)
                tk |= (uint64_t)dig << shift;
            else
                tl |= (uint32_t)dig << shift;
            done = pick[2] == need;   // the whole bin is taken: the rest of T stays 0
        }
    }
    // selected: composite >= T, and not an empty slot (composite 0)
    bool sel[E];
    uint64_t bal[E];
#pragma unroll
    for (int e = 0; e < E; e++) {
        sel[e] = (key[e] > tk || (key[e] == tk && lo[e] >= tl)) && (key[e] | lo[e]) != 0;
        bal[e] = __ballot(sel[e]);
        if (lane == 0)
            off[e * kSelWaves + wave] = __popcll(bal[e]);
    }
    __syncthreads();
    // exclusive offsets in element order (slab e major, then wave), and the total at off[kSlots]
    if (wave == 0) {
        const int c0 = lane < kSlots ? off[lane] : 0;
        const int c1 = lane + 64 < kSlots ? off[lane + 64] : 0;
        int s_0 = c0, s_1 = c1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t0 = __shfl_up(s_0, d, 64), t1 = __shfl_up(s_1, d, 64);
            if (lane >= d) {
                s_0 += t0;
                s_1 += t1;
            }
        }
        const int tot0 = __shfl(s_0, 63, 64), tot1 = __shfl(s_1, 63, 64);
        if (lane < kSlots)
            off[lane] = s_0 - c0;
        if (lane + 64 < kSlots)
            off[lane + 64] = tot0 + s_1 - c1;
        if (lane == 0)
            off[kSlots] = tot0 + tot1;
    }
    __syncthreads();
    const int total = off[kSlots];
    const int64_t o_base = ids_final ? (int64_t)h * k : ((int64_t)h * gridDim.x + blockIdx.x) * k;
#pragma unroll
    for (int e = 0; e < E; e++) {
        if (sel[e]) {
            const int pos = off[e * kSelWaves + wave] +
                            (int)__builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(bal[e] >> 32),
                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal[e], 0u));
            const uint32_t id = ~lo[e];
            if (ids_final) {
                ids_final[o_base + pos] = (int32_t)id;
            } else {
                out_key[o_base + pos] = key[e];
                out_id[o_base + pos] = id;
            }
        }
    }
    for (int pos = total + tid; pos < k; pos += kSelThreads) {
        if (ids_final) {
            ids_final[o_base + pos] = -1;
        } else {
            out_key[o_base + pos] = 0;
            out_id[o_base + pos] = kNoId;
        }
    }
}

// Candidate entries per head after each selection level, for n input elements.
inline int64_t sel_level_out(int64_t n, int k)
{
    const int64_t seg = (int64_t)sel_seg_e(k) * kSelThreads;
    return (n + seg - 1) / seg * k;
}

}  // namespace

extern "C" size_t kvt_index_topk_ws_bytes(int64_t n_blocks, int32_t n_sel, int32_t k)
{
    if (n_blocks < 0 || n_sel < 1 || k < 1)
        return 0;
    if (k <= kWaveK) {
        const size_t c = (size_t)n_sel * (size_t)std::max<int64_t>((n_blocks + kScoreRows - 1) / kScoreRows, 1) * k;
        return round_up(c * 8, 256) + round_up(c * 4, 256) + 256;
    }
    // rank keys of every block, then two ping-pong candidate buffers (key + id)
    const size_t keys = (size_t)n_sel * (size_t)std::max<int64_t>(n_blocks, 1);
    const int64_t a = n_blocks > kSelFinalE * kSelThreads ? sel_level_out(n_blocks, k) : 0;
    const int64_t b = a > kSelFinalE * kSelThreads ? sel_level_out(a, k) : 0;
    const size_t ca = (size_t)n_sel * (size_t)a, cb = (size_t)n_sel * (size_t)b;
    return round_up(keys * 8, 256) + round_up(ca * 8, 256) + round_up(ca * 4, 256) +
           round_up(cb * 8, 256) + round_up(cb * 4, 256) + 256;
}

// S3+S4: QSA-KVO pooled-plane scoring and top-k block selection.
extern "C" int kvt_index_topk(const void *pooled, int64_t n_blocks, int32_t dim,
                              const void *q_idx, int32_t n_sel, int32_t k, int32_t *ids,
                              double *scores, void *ws, size_t ws_bytes, void *stream)
{
    if (n_blocks < 0 || n_blocks > 0x7fffffffll || dim < 8 || dim > 256 || dim % 8 ||
        n_sel < 1 || n_sel > 32 || k < 1 || k > 2048)
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
        const int64_t n_wg = (n_blocks + kScoreRows - 1) / kScoreRows;   // one list per head each
        const size_t c = (size_t)n_sel * (size_t)std::max<int64_t>(n_wg, 1) * k;
        uintptr_t w = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
        uint64_t *ck = reinterpret_cast<uint64_t *>(w);
        uint32_t *ci = reinterpret_cast<uint32_t *>(w + round_up(c * 8, 256));
        if (n_wg > 0) {
            using Sh = ScoreShape<false>;
            const unsigned grid = (unsigned)n_wg * (unsigned)((n_sel + Sh::kHeads - 1) / Sh::kHeads);
            hipLaunchKernelGGL(score_wave_topk<false>, dim3(grid), dim3(Sh::kThreads), Sh::lds_bytes(dim), s,
                               static_cast<const uint16_t *>(pooled), n_blocks, dim,
                               static_cast<const uint16_t *>(q_idx), n_sel, k, ck, ci, scores, 0.0f);
            KVT_LAUNCHED("score_wave_topk");
        }
        if (n_wg <= 32)
            hipLaunchKernelGGL(merge_wave_topk<8>, dim3(n_sel), dim3(8 * 64), 0, s, ck, ci,
                               (int)n_wg, k, ids);
        else
            hipLaunchKernelGGL(merge_wave_topk<16>, dim3(n_sel), dim3(16 * 64), 0, s, ck, ci,
                               (int)n_wg, k, ids);
        KVT_LAUNCHED("merge_wave_topk");
        return KVT_OK;
    }
    // selection path: every rank key, then exact selection levels
    uintptr_t w = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
    const size_t keys = (size_t)n_sel * (size_t)std::max<int64_t>(n_blocks, 1);
    const int64_t na = n_blocks > kSelFinalE * kSelThreads ? sel_level_out(n_blocks, k) : 0;
    const int64_t nb = na > kSelFinalE * kSelThreads ? sel_level_out(na, k) : 0;
    uint64_t *all_key = reinterpret_cast<uint64_t *>(w); w += round_up(keys * 8, 256);
    uint64_t *a_key = reinterpret_cast<uint64_t *>(w); w += round_up((size_t)n_sel * na * 8, 256);
    uint32_t *a_id = reinterpret_cast<uint32_t *>(w); w += round_up((size_t)n_sel * na * 4, 256);
    uint64_t *b_key = reinterpret_cast<uint64_t *>(w); w += round_up((size_t)n_sel * nb * 8, 256);
    uint32_t *b_id = reinterpret_cast<uint32_t *>(w);
    if (n_blocks > 0) {
        using Sh = ScoreShape<true>;
        const int64_t n_wg = (n_blocks + Sh::kRows - 1) / Sh::kRows;
        const unsigned grid = (unsigned)n_wg * (unsigned)((n_sel + Sh::kHeads - 1) / Sh::kHeads);
        hipLaunchKernelGGL(score_wave_topk<true>, dim3(grid), dim3(Sh::kThreads), Sh::lds_bytes(dim), s,
                           static_cast<const uint16_t *>(pooled), n_blocks, dim,
                           static_cast<const uint16_t *>(q_idx), n_sel, k, all_key, nullptr,
                           scores, 0.0f);
        KVT_LAUNCHED("score_wave_topk");
    }
    const uint64_t *in_key = all_key;
    const uint32_t *in_id = nullptr;
    int64_t n = n_blocks;
    bool to_a = true;
    while (n > kSelFinalE * kSelThreads) {
        const int e = sel_seg_e(k);
        const int64_t segs = (n + (int64_t)e * kSelThreads - 1) / ((int64_t)e * kSelThreads);
        uint64_t *ok = to_a ? a_key : b_key;
        uint32_t *oi = to_a ? a_id : b_id;
        if (e == 8)
            hipLaunchKernelGGL(select_level<8>, dim3((unsigned)segs, n_sel), dim3(kSelThreads),
                               0, s, in_key, in_id, n, k, ok, oi, nullptr);
        else
            hipLaunchKernelGGL(select_level<4>, dim3((unsigned)segs, n_sel), dim3(kSelThreads),
                               0, s, in_key, in_id, n, k, ok, oi, nullptr);
        KVT_LAUNCHED("select_level");
        in_key = ok;
        in_id = oi;
        n = segs * k;
        to_a = !to_a;
    }
    // the last level: the smaller form when the candidates fit it
    if (n <= 4 * kSelThreads)
        hipLaunchKernelGGL(select_level<4>, dim3(1, n_sel), dim3(kSelThreads), 0, s, in_key, in_id,
                           n, k, nullptr, nullptr, ids);
    else
        hipLaunchKernelGGL(select_level<kSelFinalE>, dim3(1, n_sel), dim3(kSelThreads), 0, s,
                           in_key, in_id, n, k, nullptr, nullptr, ids);
    KVT_LAUNCHED("select_level");
    return KVT_OK;
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
