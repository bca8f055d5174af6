// Device code of the speculative-decoding verifier for gfx950 (CDNA4).
//
// Method: the spec-decoding page at dpshk.com/news/5598276 ("企业官网建设流程全解析"),
// sections 3.1-3.2 (accept with probability min(1, p/q), stop at the first
// rejection, redraw from (p - q)_+), 5.2 (q floored at 1e-10, strict
// comparison of the uniform with the accept probability, prefix acceptance), 5.3 (bonus token from the
// last target row) and 8 (T = 0 is greedy).
//
// Two kernels per verify step, both bandwidth-bound streams over the vocabulary:
//
//   rows kernel  streams every target row once with 16-byte loads (two batches
//                of loads in flight per thread), keeping a per-thread online max
//                and sum of exp2((l - m) * log2(e) / T) (fp32 exponentials summed
//                into fp64), or a running argmax for greedy rows; reduces across
//                the 64-wide waves with DPP lane moves and across the four waves
//                through LDS, and stores one partial per (row, piece), plus the
//                row's drafted token (id, logit, q) from its piece 0.  When rows
//                are 16-byte aligned the flattened [rows x vocab] stream is cut
//                into equal contiguous ranges, one per workgroup (a range covers
//                pieces of one or two rows); otherwise each row is cut into equal
//                splits with scalar head/tail handling.  No workgroup waits on
//                another: the launch boundary orders these stores before the
//                draw kernel.
//   draw kernel  every workgroup of a request first resolves it: thread i merges
//                row i's pieces, runs its accept test, and the first rejection k
//                is found with a ballot; workgroup 0 writes the outputs.  Then the
//                draw row of a sampled request (residual (p - q)_+ at k, or bonus
//                p) is streamed in fp64, one or two 2048-token blocks per wave,
//                with per-block sums; the last workgroup of the request rebuilds
//                the exact fp64 normaliser, picks the block holding v * S by a
//                block scan, rescans that block token by token and writes the
//                token.
//
// The draw kernel's arrival counters are reset by their last arrival, so every
// call leaves the scratch ready for the next.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace sv {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));   // one 16-byte load

constexpr int kThreads = 256;            // 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kRowUnroll = 4;            // 16-byte vectors per thread per batch (two batches in flight)
constexpr int kMaxPieces = 64;           // partials per row (at most one per merging thread)
// A draw block is 2048 consecutive tokens of a draw row, worked on by one wave:
// four sub-blocks of 512 tokens, lane L holding tokens 8L .. 8L+7 of each, so
// every 16-byte load instruction of the wave reads one contiguous span.
constexpr int kSubTokens = 8;                        // tokens per lane per sub-block
constexpr int kSubBlocks = 4;
constexpr int kSubElems = 64 * kSubTokens;           // 512
constexpr int kBlockElems = kSubBlocks * kSubElems;  // 2048
constexpr int kMaxDrawBlocks = 256;                  // vocab up to 2^19 tokens
constexpr int kMaxVocab = kMaxDrawBlocks * kBlockElems;   // 524288
constexpr int kSelPer = kMaxDrawBlocks / 64;         // blocks per lane in the select
constexpr int kMarginSlots = 2;          // marginal tokens kept inline per block record (code assumes 2)
constexpr double kLog2e = 1.4426950408889634;
constexpr double kQFloor = 1e-10;        // page section 5.2: q is floored at 1e-10 before dividing
// Relative margin within which a residual weight's sign could depend on the
// last bits of the normaliser; such tokens are kept aside and re-evaluated with
// the exact fp64 normaliser.
constexpr double kSignMargin = 1e-5;

enum : int { kDrawNone = 0, kDrawResidual = 1, kDrawBonus = 2, kDrawDegenerate = 3 };
enum : uint32_t { kErrDraftId = 1u, kErrOffsets = 2u, kErrNonFinite = 4u, kErrTopk = 16u };
// How q is given: dense rows [D, V]; sparse (id, prob) entries [D, topk] with q = 0
// off the list; or a point mass at the drafted token (q(x_i) = 1, a draft proposed
// without a draft model).
enum : int { kQDense = 0, kQSparse = 1, kQPoint = 2 };

struct Piece {           // one (row, piece) partial
    float m;             // piece max of the raw logits (or the argmax value)
    int g;               // piece argmax (greedy rows)
    double z;            // sum of exp2((l - m) * c) over the piece
};

struct RowStat {         // merged statistics of one target row
    float m;             // max raw logit
    int g;               // argmax (greedy rows), -1 otherwise
    double z;            // normaliser Z (fp32 exponentials, fp64 sum)
    float lx;            // logit of the drafted token of this position
    float qx;            // q of the drafted token
    int x;               // drafted token, -1 if invalid / none
    int np;              // pieces of the row (stored by its piece 0)
};

struct DrawTask {        // written by the resolving workgroup, read by the draw kernel
    int kind;            // kDraw*
    int row;             // target row holding the draw distribution
    int drow;            // draft row of q (residual only)
    int pos;             // output column k
    float v;             // uniform of the draw
    float m;             // the draw row's max logit
    double z32;          // the draw row's normaliser (fp32 exponentials)
};

struct BlockRec {        // per (request, draw block) sums
    double se;           // sum of e = exp((l - m) / T) in fp64
    double ea;           // sum of e over tokens whose residual is clearly positive
    double qa;           // sum of q over the same tokens
    int nm;              // tokens whose residual sign is marginal
    int mx[kMarginSlots];        // their ids (first kMarginSlots, in token order)
    float mq[kMarginSlots];      // their q
    int pad;
    double me[kMarginSlots];     // their e
};

struct Params {
    // problem
    const void* logits;
    const float* q;
    const int32_t* ids;
    const float* temperature;
    const float* uniforms;
    const int32_t* offsets;
    int32_t* out_tokens;
    int32_t* out_num;
    float* diag_m;
    double* diag_z;
    float* diag_r;
    int qmode;                 // kQ*
    int topk;                  // entries per sparse q row
    const int32_t* topk_ids;   // [D, topk]
    const float* topk_probs;   // [D, topk]
    uint32_t* stats;           // optional acceptance counters
    int batch, gamma, total_draft, vocab;
    // launch geometry
    int splits;          // split rows kernel: workgroups per row
    long flat_nv;        // flat rows kernel: total 16-byte vectors
    long flat_vpr;       // flat rows kernel: vectors per row
    int draw_wgs;        // draw kernel: workgroups per request
    int draw_cmajor;     // draw kernel: workgroup w serves request w % batch (else w / draw_wgs)
    int rows_grid;       // flat rows kernel: its grid
    int max_pieces;      // most pieces any row is cut into (either rows kernel)
    double flat_inv_nv, flat_inv_vpr, flat_inv_grid;   // 1 / flat_nv, 1 / flat_vpr, 1 / rows_grid
    int nblocks;         // draw blocks per row
    // scratch
    Piece* parts;        // [rows][kMaxPieces]
    RowStat* rows;
    BlockRec* recs;
    uint32_t* draw_cnt;
    uint32_t* err;       // sticky contract-violation word (device)
    uint32_t* err_host;  // host-mapped copy the host checks before a call, or nullptr
};

// ----------------------------------------------------------------- element types
struct F32 {
    using T = float;
    static constexpr int kPerVec = 4;
    static __device__ __forceinline__ void decode(const v4u& v, float* f) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    static __device__ __forceinline__ float load1(const void* row, long x) {
        return static_cast<const float*>(row)[x];
    }
    static __device__ __forceinline__ uint32_t bits1(const void* row, long x) {
        return static_cast<const uint32_t*>(row)[x];
    }
    static __device__ __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b); }
    static constexpr int kBits = 32;
    static constexpr uint32_t kNegInfBits = 0xff800000u;
    static constexpr uint32_t kNegInfWord = 0xff800000u;
};

struct BF16 {
    using T = uint16_t;
    static constexpr int kPerVec = 8;
    static __device__ __forceinline__ void decode(const v4u& v, float* f) {
        f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
        f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
        f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
    }
    static __device__ __forceinline__ float load1(const void* row, long x) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[x]) << 16);
    }
    static __device__ __forceinline__ uint32_t bits1(const void* row, long x) {
        return static_cast<uint32_t>(static_cast<const uint16_t*>(row)[x]);
    }
    static __device__ __forceinline__ float from_bits(uint32_t b) { return __uint_as_float(b << 16); }
    static constexpr int kBits = 16;
    static constexpr uint32_t kNegInfBits = 0xff80u;
    static constexpr uint32_t kNegInfWord = 0xff80ff80u;
};

// ----------------------------------------------------------------- cross-workgroup hand-off
// gfx950 has one L2 per XCD and the L2s are not coherent with each other.  A
// C++ release/acquire at agent scope therefore writes back and invalidates the
// whole L2 of the issuing XCD, which costs microseconds and would be paid by
// thousands of workgroups per call.  The hand-off here avoids it: data another
// workgroup will read is written with device-scope stores (written through to
// the device-coherent level) and read with device-scope loads; every writing
// wave waits for its own stores to complete before the workgroup bumps an
// arrival counter, and the counter RMW is performed at the device-coherent
// level.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <typename T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coherent(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t arrive(uint32_t* cnt) {
    wait_stores();
    return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t arrive_n(uint32_t* cnt, uint32_t n) {
    wait_stores();
    return __hip_atomic_fetch_add(cnt, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t* cnt) {
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A counter bumped at the device-coherent level (its result is not used).
__device__ __forceinline__ void count_add(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Sets contract-violation bits in the sticky device word and, when the caller
// gave one, in the host-mapped word the host checks at its next call (a
// system-scope store of the word's new value; rare path).
__device__ __forceinline__ void flag_error(uint32_t* err, uint32_t* err_host, uint32_t bits) {
    const uint32_t old = __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (err_host) __hip_atomic_store(err_host, old | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ----------------------------------------------------------------- fp64 exp2
// kExp2Table[j] = 2^(j/1024), j = 0..1023 (generated by gen_exp2_table.py).
#include "sv_exp2_table.h"
constexpr int kExp2TableSize = 1024;
constexpr int kExp2Shift = 10;               // log2 of the table size
constexpr double kExp2Scale = 1024.0;        // exp2_tab takes its argument times this
// Adding 1.5 * 2^52 to a double of magnitude below 2^51 rounds it to an integer
// (to nearest, ties to even) that then sits in the low bits of the mantissa.
constexpr double kRoundMagic = 6755399441055744.0;

// 2^(s/1024) for s <= 0 (s = -inf allowed), relative error below 1e-15: s = k + r
// with |r| <= 1/2 exactly (k rounded by the magic addition, whose low word is k
// itself), 2^(r/1024) by its Taylor series in r*ln2/1024 to degree 3 (truncation
// below 5.5e-16; the coefficients are (ln2)^i / i! scaled by 2^(-10i), exactly),
// 2^((k mod 1024)/1024) from the table (kept in LDS by the caller) and
// 2^(k div 1024) by ldexp.  s is clamped at -1105920 = 1024 * -1080 first, whose
// power of two is below the smallest double, so such results (and NaN inputs)
// are 0.  Taking s already scaled by 1024 (folded into the caller's
// coefficients, exactly) keeps the rounding to one add; the 1024-entry table
// keeps the polynomial one fma shorter than a 256-entry one would.
__device__ __forceinline__ double exp2_tab(double s, const double* tab) {
    s = fmax(s, -1105920.0);
    const double t = s + kRoundMagic;
    const int k = __double2loint(t);
    const double r = s - (t - kRoundMagic);
    double p = fma(r, 5.1692229383458926e-11, 2.2909784980688164e-07);
    p = fma(r, p, 0.0006769015435155716);
    p = fma(r, p, 1.0);
    return ldexp(tab[k & (kExp2TableSize - 1)] * p, k >> kExp2Shift);
}

// ----------------------------------------------------------------- reductions
// Wave reductions use DPP lane moves inside each 16-lane row (quad swaps, then
// the half-row and row mirrors, after which every lane of a row holds the row's
// result) and combine the four rows in a fixed order with readlane, so every
// lane receives the same value.
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, Ctrl, RowMask, 0xf, false);
}
template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(dpp_i<Ctrl, RowMask>(__float_as_int(old), __float_as_int(v)));
}
template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ double dpp_d(double old, double v) {
    const long long o = __double_as_longlong(old), x = __double_as_longlong(v);
    const int lo = dpp_i<Ctrl, RowMask>(static_cast<int>(o), static_cast<int>(x));
    const int hi = dpp_i<Ctrl, RowMask>(static_cast<int>(o >> 32), static_cast<int>(x >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ __forceinline__ int rdlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float rdlane(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
__device__ __forceinline__ double rdlane(double v, int l) {
    const long long x = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(x), l);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(x >> 32), l);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// Row-wide combine with op (all 16 lanes of a row end with the row result),
// then the four rows in order 0, 1, 2, 3.
#define SV_WAVE_REDUCE(T, DPP, OP, v)                                   \
    do {                                                                \
        v = OP(v, DPP<kDppQuadSwap1>(v, v));                            \
        v = OP(v, DPP<kDppQuadSwap2>(v, v));                            \
        v = OP(v, DPP<kDppRowHalfMirror>(v, v));                        \
        v = OP(v, DPP<kDppRowMirror>(v, v));                            \
        const T r0 = rdlane(v, 15), r1 = rdlane(v, 31), r2 = rdlane(v, 47), r3 = rdlane(v, 63); \
        v = OP(OP(OP(r0, r1), r2), r3);                                 \
    } while (0)

__device__ __forceinline__ float op_maxf(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ double op_addd(double a, double b) { return a + b; }
__device__ __forceinline__ int op_addi(int a, int b) { return a + b; }
__device__ __forceinline__ int op_mini(int a, int b) { return min(a, b); }
__device__ __forceinline__ int op_maxi(int a, int b) { return max(a, b); }

__device__ __forceinline__ float wave_max(float v) {
    SV_WAVE_REDUCE(float, dpp_f, op_maxf, v);
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
    SV_WAVE_REDUCE(double, dpp_d, op_addd, v);
    return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
    SV_WAVE_REDUCE(int, dpp_i, op_addi, v);
    return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
    SV_WAVE_REDUCE(int, dpp_i, op_mini, v);
    return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
    SV_WAVE_REDUCE(int, dpp_i, op_maxi, v);
    return v;
}
// (value, index) argmax: larger value wins, lower index on ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
template <int Ctrl>
__device__ __forceinline__ void argmax_dpp_step(float& v, int& i) {
    const float v2 = dpp_f<Ctrl>(v, v);
    const int i2 = dpp_i<Ctrl>(i, i);
    argmax_merge(v, i, v2, i2);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_dpp_step<kDppQuadSwap1>(v, i);
    argmax_dpp_step<kDppQuadSwap2>(v, i);
    argmax_dpp_step<kDppRowHalfMirror>(v, i);
    argmax_dpp_step<kDppRowMirror>(v, i);
    float rv = rdlane(v, 15);
    int ri = rdlane(i, 15);
    argmax_merge(rv, ri, rdlane(v, 31), rdlane(i, 31));
    argmax_merge(rv, ri, rdlane(v, 47), rdlane(i, 47));
    argmax_merge(rv, ri, rdlane(v, 63), rdlane(i, 63));
    v = rv;
    i = ri;
}
// Inclusive prefix sum over the wave's lanes (row shifts 1, 2, 4, 8, then the
// row broadcasts 15 and 31).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
    v += dpp_d<kDppRowShr1>(0.0, v);
    v += dpp_d<kDppRowShr1 + 1>(0.0, v);
    v += dpp_d<kDppRowShr1 + 3>(0.0, v);
    v += dpp_d<kDppRowShr1 + 7>(0.0, v);
    v += dpp_d<kDppRowBcast15, 0xa>(0.0, v);
    v += dpp_d<kDppRowBcast31, 0xc>(0.0, v);
    return v;
}

// Workgroup reductions: every thread receives the result (fixed combination order).
struct RedScratch {
    float f[kWaves];
    double d[kWaves];
    int i[kWaves];
    int o0, o1;          // map_row: the found request's offsets and temperature,
    float T;             // passed on by the thread that loaded them
};

__device__ __forceinline__ float wg_max(float v, RedScratch& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) s.f[w] = v;
    __syncthreads();
    float r = s.f[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = fmaxf(r, s.f[k]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ double wg_sum(double v, RedScratch& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_sum(v);
    if (lane == 0) s.d[w] = v;
    __syncthreads();
    double r = s.d[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r += s.d[k];
    __syncthreads();
    return r;
}
__device__ __forceinline__ int wg_sum_int(int v, RedScratch& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_sum_int(v);
    if (lane == 0) s.i[w] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) r += s.i[k];
    __syncthreads();
    return r;
}
__device__ __forceinline__ int wg_min_int(int v, RedScratch& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_min_int(v);
    if (lane == 0) s.i[w] = v;
    __syncthreads();
    int r = s.i[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = min(r, s.i[k]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ int wg_max_int(int v, RedScratch& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_max_int(v);
    if (lane == 0) s.i[w] = v;
    __syncthreads();
    int r = s.i[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = max(r, s.i[k]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ void wg_argmax(float& v, int& i, RedScratch& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    wave_argmax(v, i);
    if (lane == 0) { s.f[w] = v; s.i[w] = i; }
    __syncthreads();
    float rv = s.f[0];
    int ri = s.i[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) argmax_merge(rv, ri, s.f[k], s.i[k]);
    __syncthreads();
    v = rv; i = ri;
}
// Inclusive prefix sum over the workgroup (thread order); also returns the total.
__device__ __forceinline__ double wg_inclusive_scan(double v, double& total, RedScratch& s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_inclusive_scan(v);
    if (lane == 63) s.d[w] = v;
    __syncthreads();
    double before = 0.0, tot = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        if (k < w) before += s.d[k];
        tot += s.d[k];
    }
    __syncthreads();
    total = tot;
    return before + v;
}

// ----------------------------------------------------------------- request lookup
// Maps target row t to (request b, position i, gamma_b, first draft row).
struct RowMap {
    int b, i, gb, d0;
    bool ok;
    float T;             // the request's temperature
};

__device__ __forceinline__ RowMap map_row(const Params& P, int t, RedScratch& red) {
    RowMap r;
    if (P.offsets == nullptr) {
        r.b = t / (P.gamma + 1);
        r.i = t - r.b * (P.gamma + 1);
        r.gb = P.gamma;
        r.d0 = r.b * P.gamma;
        r.ok = true;
        r.T = P.temperature[r.b];
        return r;
    }
    // Request b starts at target row offsets[b] + b: count the starts <= t.  In
    // the same round of loads each thread keeps the offsets and temperature of
    // the last request whose start it counted; the thread that counted b's start
    // passes them on through LDS between the sum's two barriers, so no second
    // round trip follows.  With inconsistent offsets no thread may own b: the
    // sentinel then fails the checks below.
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) red.o0 = -1;
    int cnt = 0, jmax = -1, oj0 = 0, oj1 = 0;
    float tj = 0.0f;
    for (int j = threadIdx.x; j < P.batch; j += kThreads) {
        const int o = P.offsets[j];
        const int on = P.offsets[j + 1];
        const float tt = P.temperature[j];
        if (o + j <= t) {
            ++cnt;
            jmax = j;
            oj0 = o;
            oj1 = on;
            tj = tt;
        }
    }
    cnt = wave_sum_int(cnt);
    if (lane == 0) red.i[w] = cnt;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) total += red.i[k];
    const int b = total - 1;
    if (jmax >= 0 && jmax == b) {
        red.o0 = oj0;
        red.o1 = oj1;
        red.T = tj;
    }
    __syncthreads();
    const int o0 = red.o0, o1 = red.o1;
    r.b = b;
    r.T = red.T;
    r.gb = o1 - o0;
    r.d0 = o0;
    r.i = t - (o0 + b);
    r.ok = (b >= 0) && (b < P.batch) && (o0 >= 0) && (o1 <= P.total_draft) && (r.gb >= 0) &&
           (r.gb <= P.gamma) && (r.i >= 0) && (r.i <= r.gb);
    // uniform: a failing caller returns at once, and this barrier keeps the
    // fields above from being overwritten by its next lookup before every
    // thread has read them (a passing caller reduces over the workgroup first)
    if (!r.ok) __syncthreads();
    return r;
}

// ----------------------------------------------------------------- row streaming
struct RowShared {
    RedScratch red;
    int flag;
    int k;
    float mk;            // resolve: statistics of row k for the draw task
    double zk;
};

// Per-thread online max and sum over one batch of decoded logits.  The sum is
// kept against a reference kref, an integer in log2 units, as
// st = sum 2^(l c - kref): kref moves up (to ceil of the batch max times c)
// only when the batch max times c passes it by more than kRefSlack, and the sum
// is then rescaled by an exact power of two.  Terms are at most 2^kRefSlack, and
// the common path is one fma, one exp2 and one add per logit.  mt is the exact
// running max.  kRefStart makes the first finite batch set the reference, and
// turns -inf logits into zero terms.
constexpr float kRefSlack = 8.0f;
constexpr float kRefStart = -1e30f;
template <int N>
__device__ __forceinline__ void accumulate_batch(const float* f, float c, float& mt, float& kref, double& st) {
    float bm = f[0];
#pragma unroll
    for (int k = 1; k < N; ++k) bm = fmaxf(bm, f[k]);
    mt = fmaxf(mt, bm);
    const float bmc = bm * c;
    if (bmc > kref + kRefSlack) {
        const float knew = ceilf(bmc);
        st = ldexp(st, static_cast<int>(fmaxf(kref - knew, -2048.0f)));
        kref = knew;
    }
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < N; ++k) acc += __builtin_amdgcn_exp2f(fmaf(f[k], c, -kref));
    st += static_cast<double>(acc);
}

// Argmax over one loaded batch (vectors jb .. jb + kRowUnroll - 1 of this
// thread's n), element indices counted from the row start.  A thread visits its
// elements in increasing index order, so a strictly greater value is the only
// one that replaces the running argmax (the lowest index wins a tie); the
// reductions across lanes and pieces break ties by index.
template <typename E>
__device__ __forceinline__ void argmax_batch(const v4u* buf, int jb, int n, long first, int head, float& bv, int& bi) {
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
        float f[E::kPerVec];
        E::decode(buf[u], f);
        const int x0 = head + static_cast<int>((first + (long)(jb + u) * kThreads) * E::kPerVec);
        if (jb + u < n) {
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) {
                const bool gt = f[k] > bv;
                bv = gt ? f[k] : bv;
                bi = gt ? x0 + k : bi;
            }
        }
    }
}

// One batch: vectors first + u * kThreads for u < count (count >= 1).  Every
// load is issued, the ones past the range from vector `first` itself, so that
// no branch surrounds a load and the compiler can wait for exactly one batch;
// the consumer replaces the surplus values (mask_batch) when it takes the batch
// in, after the next batch's loads are on their way.
template <typename E>
__device__ __forceinline__ void load_batch(v4u* buf, const v4u* vp, long first, int count) {
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
        const long idx = (u < count) ? first + (long)u * kThreads : first;
        buf[u] = __builtin_nontemporal_load(vp + idx);
    }
}
template <typename E>
__device__ __forceinline__ void mask_batch(v4u* buf, int count) {
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u)
        if (u >= count) buf[u] = v4u(E::kNegInfWord);
}
// Takes a loaded batch (count of its vectors in range) into the running sums;
// kFull: the caller knows every vector of the batch is in range (no masking).
template <typename E, bool kFull = false>
__device__ __forceinline__ void take_batch(v4u* buf, int count, float c, float& mt, float& kref, double& st) {
    if (!kFull) mask_batch<E>(buf, count);
    float f[kRowUnroll * E::kPerVec];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) E::decode(buf[u], f + u * E::kPerVec);
    accumulate_batch<kRowUnroll * E::kPerVec>(f, c, mt, kref, st);
}

// The drafted token of a target row, read by every piece of the row (thread 0)
// so that whichever workgroup merges the row has it at hand: its id, logit and
// q (x = -1: no drafted token here, or an id outside the vocabulary).
struct DraftTok {
    int x = -1;
    float lx = 0.0f, qx = 0.0f;
};

// Streams vectors [v0, v1) of target row t (vectors counted from the row's first
// 16-byte aligned element), adds the scalar head (piece 0) and tail (last piece)
// and stores the piece; the row's piece 0 also stores the drafted token's id,
// logit and q for the draw kernel's resolve (x = -2 marks a draft row whose
// sparse q breaks the contract: an entry id outside [-1, vocab) or the drafted
// token listed twice).  The first batch of loads is issued before the request
// lookup, and the drafted token's logit and q are read once the stream has been
// taken in, both so that their round trips overlap other work.  No arrival is
// counted: the launch boundary orders these stores before the next kernel.
// Issue priority of a streaming wave: 3 over its workgroup's first quarter of
// vectors down to 0 over the last.  A CU otherwise issues for its oldest waves
// first, so its workgroups would finish in dispatch order and the last one
// would stream alone with a third of the loads in flight; with the priority
// falling as a wave advances, the waves that are behind are served first and
// the workgroups of a CU end together.
__device__ __forceinline__ void set_stream_priority(int level) {
    if (level >= 3) __builtin_amdgcn_s_setprio(3);
    else if (level == 2) __builtin_amdgcn_s_setprio(2);
    else if (level == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// done0 / total: vectors of the workgroup's range before this piece / in the
// whole range (total 0: the piece is the range).
template <typename E>
__device__ __forceinline__ void row_piece_publish(const Params& P, int t, long v0, long v1, int piece, int npieces,
                                                 RowShared& sh, DraftTok& dt, long done0 = 0, long total = 0) {
    const int tid = threadIdx.x;
    const int V = P.vocab;

    const typename E::T* row = static_cast<const typename E::T*>(P.logits) + (size_t)t * V;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
    int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(typename E::T));
    if (head > V) head = V;
    const long nvec = (V - head) / E::kPerVec;
    const int tail = V - head - static_cast<int>(nvec * E::kPerVec);
    const v4u* vp = reinterpret_cast<const v4u*>(row + head);

    // this thread's vectors: v0 + tid + 256 j, j < n
    const long span = v1 - v0 - tid;
    const int n = span > 0 ? static_cast<int>((span + kThreads - 1) / kThreads) : 0;
    const long first = v0 + tid;
    v4u A[kRowUnroll];
    if (n > 0) load_batch<E>(A, vp, first, n);

    const RowMap rm = map_row(P, t, sh.red);
    if (!rm.ok) {
        if (tid == 0 && piece == 0) flag_error(P.err, P.err_host, kErrOffsets);
        return;
    }
    const int i = rm.i, gb = rm.gb;
    const float T = rm.T;
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : static_cast<float>(kLog2e / static_cast<double>(T));
    int xd = -1;
    if (tid == 0 && !greedy && i < gb && piece == 0) xd = P.ids[rm.d0 + i];

    // the batches at which the range's second, third and last quarters start
    const long range = total > 0 ? total : v1 - v0;
    constexpr int kBatchVecs = kRowUnroll * kThreads;
    const int q1 = static_cast<int>((range / 4 - done0) / kBatchVecs);
    const int q2 = static_cast<int>((range / 2 - done0) / kBatchVecs);
    const int q3 = static_cast<int>((3 * range / 4 - done0) / kBatchVecs);

    float mloc;          // piece max (sampled) / argmax value (greedy)
    int gloc = -1;       // argmax (greedy)
    double zloc = 0.0;   // piece sum (sampled)
    if (!greedy) {
        float mt = -INFINITY, kref = kRefStart;
        double st = 0.0;
        v4u Bf[kRowUnroll];
        // batch j holds this thread's vectors j * kRowUnroll ...; A holds batch 0.
        // Steady state: two batches at a time with every load unconditional, so
        // the next batch is always in flight while one is taken in; then the
        // last one or two batches.
        const int nb = (n + kRowUnroll - 1) / kRowUnroll;
        int j = 0;
        // (batches j and j + 1 come before the last batch here, so they are full)
        for (; j + 2 < nb; j += 2) {
            set_stream_priority(3 - static_cast<int>(j >= q1) - static_cast<int>(j >= q2) - static_cast<int>(j >= q3));
            load_batch<E>(Bf, vp, first + (long)(j + 1) * kRowUnroll * kThreads, n - (j + 1) * kRowUnroll);
            take_batch<E, true>(A, kRowUnroll, c, mt, kref, st);
            load_batch<E>(A, vp, first + (long)(j + 2) * kRowUnroll * kThreads, n - (j + 2) * kRowUnroll);
            take_batch<E, true>(Bf, kRowUnroll, c, mt, kref, st);
        }
        if (j + 1 < nb) {
            load_batch<E>(Bf, vp, first + (long)(j + 1) * kRowUnroll * kThreads, n - (j + 1) * kRowUnroll);
            take_batch<E>(A, n - j * kRowUnroll, c, mt, kref, st);
            take_batch<E>(Bf, n - (j + 1) * kRowUnroll, c, mt, kref, st);
        } else if (j < nb) {
            take_batch<E>(A, n - j * kRowUnroll, c, mt, kref, st);
        }
        __builtin_amdgcn_s_setprio(0);
        dt.x = -1;
        if (tid == 0 && xd >= 0 && xd < V) {
            dt.x = xd;
            dt.lx = E::load1(row, xd);
            dt.qx = (P.qmode == kQDense) ? P.q[(size_t)(rm.d0 + i) * V + xd] : 1.0f;
        }
        if (P.qmode == kQSparse && i < gb && piece == 0 && tid < 64) {
            // wave 0 of the row's piece 0 looks the drafted token up in its row's
            // entries (absent: q = 0) and checks every entry id
            const int xw = __builtin_amdgcn_readfirstlane(xd);
            float qv = 0.0f;
            if (xw >= 0 && xw < V) {
                const size_t e0 = (size_t)(rm.d0 + i) * P.topk;
                const int id = tid < P.topk ? P.topk_ids[e0 + tid] : -1;
                const float pr = tid < P.topk ? P.topk_probs[e0 + tid] : 0.0f;
                const unsigned long long hit = __ballot(id == xw);
                const unsigned long long bad = __ballot(id < -1 || id >= V);
                if (hit != 0ull) qv = rdlane(pr, __ffsll(static_cast<long long>(hit)) - 1);
                if (__popcll(hit) > 1 || bad != 0ull) {
                    if (tid == 0) flag_error(P.err, P.err_host, kErrTopk);
                    dt.x = -2;
                }
            }
            if (tid == 0) dt.qx = qv;
        }
        // unaligned head (piece 0) and tail (last piece): at most 7 scalars each
        float fx = -INFINITY;
        if (piece == 0 && tid < head) fx = E::load1(row, tid);
        if (piece == npieces - 1 && tid >= 64 && tid - 64 < tail) fx = E::load1(row, head + nvec * E::kPerVec + (tid - 64));
        accumulate_batch<1>(&fx, c, mt, kref, st);

        mloc = wg_max(mt, sh.red);
        double zs = 0.0;
        if (mt > -INFINITY)
            zs = st * exp2(static_cast<double>(kref) - static_cast<double>(mloc) * static_cast<double>(c));
        zloc = wg_sum(zs, sh.red);
    } else {
        // a thread with elements starts at its first one, so that a piece of
        // -inf logits still reports its lowest index (as a tie-breaking merge would)
        float bv = -INFINITY;
        int bi = n > 0 ? head + static_cast<int>(first * E::kPerVec) : 0x7fffffff;
        dt.x = -1;
        // two batches at a time, as in the sampled stream
        v4u Bf[kRowUnroll];
        const int nb = (n + kRowUnroll - 1) / kRowUnroll;
        int j = 0;
        for (; j + 2 < nb; j += 2) {
            set_stream_priority(3 - static_cast<int>(j >= q1) - static_cast<int>(j >= q2) - static_cast<int>(j >= q3));
            load_batch<E>(Bf, vp, first + (long)(j + 1) * kRowUnroll * kThreads, n - (j + 1) * kRowUnroll);
            argmax_batch<E>(A, j * kRowUnroll, n, first, head, bv, bi);
            load_batch<E>(A, vp, first + (long)(j + 2) * kRowUnroll * kThreads, n - (j + 2) * kRowUnroll);
            argmax_batch<E>(Bf, (j + 1) * kRowUnroll, n, first, head, bv, bi);
        }
        if (j + 1 < nb) {
            load_batch<E>(Bf, vp, first + (long)(j + 1) * kRowUnroll * kThreads, n - (j + 1) * kRowUnroll);
            argmax_batch<E>(A, j * kRowUnroll, n, first, head, bv, bi);
            argmax_batch<E>(Bf, (j + 1) * kRowUnroll, n, first, head, bv, bi);
        } else if (j < nb) {
            argmax_batch<E>(A, j * kRowUnroll, n, first, head, bv, bi);
        }
        __builtin_amdgcn_s_setprio(0);
        if (piece == 0 && tid < head) argmax_merge(bv, bi, E::load1(row, tid), tid);
        if (piece == npieces - 1 && tid >= 64 && tid - 64 < tail) {
            const int x = head + static_cast<int>(nvec * E::kPerVec) + (tid - 64);
            argmax_merge(bv, bi, E::load1(row, x), x);
        }
        wg_argmax(bv, bi, sh.red);
        mloc = bv;
        gloc = bi;
    }

    // ---- publish the piece
    if (tid == 0) {
        // the launch geometry keeps piece < kMaxPieces for rows laid out as the
        // offsets promise; inconsistent offsets can break that, and are flagged
        if (piece >= kMaxPieces || npieces > kMaxPieces) {
            flag_error(P.err, P.err_host, kErrOffsets);
            return;
        }
        Piece* pp = &P.parts[(size_t)t * kMaxPieces + piece];
        st_coherent(&pp->m, mloc);
        st_coherent(&pp->g, gloc);
        st_coherent(&pp->z, zloc);
        if (piece == 0) {
            RowStat* rp = &P.rows[t];
            st_coherent(&rp->x, dt.x);
            st_coherent(&rp->lx, dt.lx);
            st_coherent(&rp->qx, dt.qx);
            st_coherent(&rp->np, npieces);
        }
    }
}

// General rows kernel: one workgroup per (target row, split); rows need not be
// 16-byte aligned.
template <typename E>
__global__ __launch_bounds__(kThreads) void rows_split_kernel(Params P) {
    __shared__ RowShared sh;
    const int S = P.splits;
    const int t = blockIdx.x / S;
    const int s = blockIdx.x - t * S;
    const int V = P.vocab;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(static_cast<const typename E::T*>(P.logits) + (size_t)t * V);
    int head = static_cast<int>(((16u - (addr & 15u)) & 15u) / sizeof(typename E::T));
    if (head > V) head = V;
    const long nvec = (V - head) / E::kPerVec;
    DraftTok dt;
    // pieces only: the draw kernel merges and resolves
    row_piece_publish<E>(P, t, (long)s * nvec / S, (long)(s + 1) * nvec / S, s, S, sh, dt);
}

// floor(x / d) for 0 <= x < 2^52 and d >= 1, given inv = 1 / d rounded to
// double.  The rounded product x * inv is within a few units in its last place
// of x / d, so its truncation is the quotient or one off it, and one step each
// way on the remainder makes it exact (the device has no integer divider; its
// software 64-bit division is a long dependent chain).
__device__ __forceinline__ long div_exact(long x, long d, double inv) {
    long q = static_cast<long>(static_cast<double>(x) * inv);
    const long r = x - q * d;
    q += (r >= d) ? 1 : 0;
    q -= (r < 0) ? 1 : 0;
    return q;
}

// Workgroup owning vector v when nv vectors are cut into g equal ranges
// [floor(w nv / g), floor((w+1) nv / g)).
__device__ __forceinline__ int range_owner(long v, long nv, int g, double inv_nv) {
    return static_cast<int>(div_exact((v + 1) * (long)g - 1, nv, inv_nv));
}

// Rows streamed only: every piece of this workgroup's range is stored
// (and each row's drafted token by its piece 0); the merges, the accept tests
// and the resolve are left to the draw kernel, which the launch boundary
// orders after every store of this one.  No workgroup waits on another.
template <typename E>
__global__ __launch_bounds__(kThreads) void rows_flat_kernel(Params P) {
    __shared__ RowShared sh;
    const int w = blockIdx.x;
    const int G = P.rows_grid;
    const long VPR = P.flat_vpr, NV = P.flat_nv;
    const long a = div_exact((long)w * NV, G, P.flat_inv_grid), e = div_exact((long)(w + 1) * NV, G, P.flat_inv_grid);
    long r = div_exact(a, VPR, P.flat_inv_vpr);
    for (long s0 = a; s0 < e; ++r) {
        const long rs = r * VPR, re = rs + VPR;
        const long s1 = e < re ? e : re;
        const int wf = range_owner(rs, NV, G, P.flat_inv_nv), wl = range_owner(re - 1, NV, G, P.flat_inv_nv);
        DraftTok dt;
        row_piece_publish<E>(P, static_cast<int>(r), s0 - rs, s1 - rs, w - wf, wl - wf + 1, sh, dt, s0 - a, e - a);
        __syncthreads();
        s0 = s1;
    }
}

// ----------------------------------------------------------------- draw blocks
// Everything a wave needs to work on one request's draw row.
template <typename E>
struct DrawRow {
    int kind;            // kDrawResidual / kDrawBonus
    int pos;             // output column
    float v;             // uniform of the draw
    double m;            // row max (raw logits)
    double c2;           // 1024 log2(e) / T
    double mc2;          // m * c2 (both exactly 1024 times their unscaled roundings)
    double z32;          // normaliser from the fp32-exponential pass
    const typename E::T* lrow;
    const float* qrow;   // residual with dense q: q row, else nullptr
    bool lalign, qalign;
    // residual with sparse or point-mass q: the block sums are those of p, and the
    // select takes the listed tokens' q off them; entry s of the draft row is
    // token sid[s] with q = sq[s] (point mass: sid = the drafted token, sq null, q = 1)
    bool qlist;
    int nq;
    const int32_t* sid;
    const float* sq;
};

// e = exp((l - m) / T) of one token, in fp64 (the same expression everywhere).
template <typename E>
__device__ __forceinline__ double draw_e(const DrawRow<E>& d, float l, const double* tab) {
    return exp2_tab(fma(static_cast<double>(l), d.c2, -d.mc2), tab);
}

// One lane's 8 tokens of one sub-block as loaded (raw element bits), and its
// 32 tokens of a whole block.
template <typename E>
struct RawSub {
    v4u l[kSubTokens / E::kPerVec];
    v4u q[kSubTokens / 4];
};
template <typename E>
struct RawBlock {
    RawSub<E> s[kSubBlocks];
};

// Loads of this lane's tokens [x0, x0 + 8) of any row: vectors where the row
// allows, else element by element (logits past V read as -inf, q as 0).
template <typename E>
__device__ __forceinline__ void issue_sub_any(const DrawRow<E>& d, long x0, int V, bool with_q, RawSub<E>& r) {
    constexpr int NL = kSubTokens / E::kPerVec;
    const bool full = x0 + kSubTokens <= V;
    if (full && d.lalign) {
        const v4u* lp = reinterpret_cast<const v4u*>(d.lrow + x0);
#pragma unroll
        for (int h = 0; h < NL; ++h) r.l[h] = __builtin_nontemporal_load(lp + h);
    } else {
        uint32_t w[4 * NL];
#pragma unroll
        for (int k = 0; k < 4 * NL; ++k) w[k] = 0u;
#pragma unroll
        for (int k = 0; k < kSubTokens; ++k) {
            const uint32_t bits = (x0 + k < V) ? E::bits1(d.lrow, x0 + k) : E::kNegInfBits;
            if (E::kBits == 16) w[k >> 1] |= bits << (16 * (k & 1));
            else w[k] = bits;
        }
#pragma unroll
        for (int h = 0; h < NL; ++h) r.l[h] = v4u{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
    }
    if (with_q) {
        if (full && d.qalign) {
            const v4u* qp = reinterpret_cast<const v4u*>(d.qrow + x0);
#pragma unroll
            for (int h = 0; h < kSubTokens / 4; ++h) r.q[h] = __builtin_nontemporal_load(qp + h);
        } else {
            uint32_t w[kSubTokens];
#pragma unroll
            for (int k = 0; k < kSubTokens; ++k) w[k] = (x0 + k < V) ? __float_as_uint(d.qrow[x0 + k]) : 0u;
#pragma unroll
            for (int h = 0; h < kSubTokens / 4; ++h) r.q[h] = v4u{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
        }
    } else {
#pragma unroll
        for (int h = 0; h < kSubTokens / 4; ++h) r.q[h] = v4u(0u);
    }
}

// This lane's first token of sub-block u of the block starting at xb.
__device__ __forceinline__ long sub_first(long xb, int u) {
    return xb + u * kSubElems + (threadIdx.x & 63) * kSubTokens;
}

// (a sub-block wholly past the row's end, in its ragged last block, is set to
// -inf logits and zero q without any load)
template <typename E>
__device__ __forceinline__ void issue_block_any(const DrawRow<E>& d, long xb, int V, bool with_q, RawBlock<E>& r) {
#pragma unroll
    for (int u = 0; u < kSubBlocks; ++u) {
        if (xb + u * kSubElems >= V) {
#pragma unroll
            for (int h = 0; h < kSubTokens / E::kPerVec; ++h) r.s[u].l[h] = v4u(E::kNegInfWord);
#pragma unroll
            for (int h = 0; h < kSubTokens / 4; ++h) r.s[u].q[h] = v4u(0u);
        } else {
            issue_sub_any<E>(d, sub_first(xb, u), V, with_q, r.s[u]);
        }
    }
}

template <typename E>
__device__ __forceinline__ void decode_sub(const RawSub<E>& r, bool with_q, float* l, float* q) {
#pragma unroll
    for (int h = 0; h < kSubTokens / E::kPerVec; ++h) E::decode(r.l[h], l + h * E::kPerVec);
#pragma unroll
    for (int h = 0; h < kSubTokens / 4; ++h) {
        if (with_q) F32::decode(r.q[h], q + 4 * h);
        else q[4 * h] = q[4 * h + 1] = q[4 * h + 2] = q[4 * h + 3] = 0.0f;
    }
}

// Token k (0..7) of a lane's loaded sub-block, decoded on its own: logit and q.
template <typename E>
__device__ __forceinline__ float sub_logit(const RawSub<E>& r, int k) {
    if (E::kBits == 16) {
        const uint32_t w = r.l[0][k >> 1];
        return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    return __uint_as_float(r.l[k >> 2][k & 3]);
}
template <typename E>
__device__ __forceinline__ float sub_q(const RawSub<E>& r, int k) {
    return __uint_as_float(r.q[k >> 2][k & 3]);
}

// Rare path of block_record: stores the block's first kMarginSlots marginal
// tokens in token order (sub-block, then lane, then position in the lane),
// reloading each from memory.  Kept out of line so that the common path's
// register allocation does not carry it.
template <typename E>
__device__ __noinline__ void record_marginal(const typename E::T* lrow, const float* qrow, double c2, double mc2,
                                             long xb, uint32_t mmask, const double* tab, BlockRec* rec) {
    const int lane = threadIdx.x & 63;
    int slot = 0;
    for (int u = 0; u < kSubBlocks && slot < kMarginSlots; ++u) {
        const uint32_t mu = (mmask >> (u * kSubTokens)) & 0xffu;
        unsigned long long lanes = __ballot(mu != 0u);
        while (lanes != 0ull && slot < kMarginSlots) {
            const int L = __ffsll(static_cast<long long>(lanes)) - 1;
            lanes &= lanes - 1ull;
            uint32_t bits = static_cast<uint32_t>(rdlane(static_cast<int>(mu), L));
            while (bits != 0u && slot < kMarginSlots) {
                const int k = __ffs(static_cast<int>(bits)) - 1;
                bits &= bits - 1u;
                if (lane == 0) {
                    const long x = xb + u * kSubElems + L * kSubTokens + k;
                    st_coherent(&rec->mx[slot], static_cast<int>(x));
                    st_coherent(&rec->mq[slot], qrow[x]);
                    st_coherent(&rec->me[slot],
                                exp2_tab(fma(static_cast<double>(E::load1(lrow, x)), c2, -mc2), tab));
                }
                ++slot;
            }
        }
    }
}

// Block sums: residual rows split the tokens three ways with the fp32-pass
// normaliser: clearly positive residual (e / Z32 * (1 - margin) > q: summed
// into ea and qa), clearly non-positive (e / Z32 * (1 + margin) <= q: dropped)
// and marginal (the rest: counted, the first kMarginSlots in token order kept
// inline).  Branch-free except for the marginal capture, which only runs when
// the wave has a marginal token.
struct BlockSums {
    double se = -0.0, ea = -0.0, qa = -0.0;   // -0.0 + x is x: the first adds fold away
    uint32_t mmask = 0u;                      // bit 8u + k: token k of sub-block u is marginal
};

// Adds one lane's 8 decoded tokens of sub-block u, two at a time.
template <typename E, bool kResidual>
__device__ __forceinline__ void accumulate_token(const DrawRow<E>& d, float l, float q, int bit, double apos,
                                                 double aneg, const double* tab, BlockSums& b) {
    const double e = draw_e<E>(d, l, tab);
    b.se += e;
    if (kResidual) {
        const double qd = static_cast<double>(q);
        const bool pos = e * apos > qd;
        const bool marg = !pos && e * aneg > qd;
        const double wpos = pos ? 1.0 : 0.0;
        b.ea = fma(e, wpos, b.ea);
        b.qa = fma(qd, wpos, b.qa);
        b.mmask |= static_cast<uint32_t>(marg) << bit;
    }
}

template <typename E, bool kResidual>
__device__ __forceinline__ void accumulate_sub(const DrawRow<E>& d, const float* l, const float* q, int u, double apos,
                                               double aneg, const double* tab, BlockSums& b) {
#pragma unroll
    for (int k = 0; k < kSubTokens; k += 2) {
        float la = l[k], lb = l[k + 1];
        // each pair starts once the previous pair is summed: the unrolled
        // chains would otherwise be interleaved before scheduling, with every
        // token's temporaries live at once
        if (k > 0) asm volatile("" : "+v"(la), "+v"(lb) : "v"(b.se));
        accumulate_token<E, kResidual>(d, la, q[k], u * kSubTokens + k, apos, aneg, tab, b);
        accumulate_token<E, kResidual>(d, lb, q[k + 1], u * kSubTokens + k + 1, apos, aneg, tab, b);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The same sums taken straight from a loaded sub-block, four (bf16) or two (fp32) tokens at a time,
// with no decoded copy of the sub-block held in registers.
template <typename E, bool kResidual>
__device__ __forceinline__ void accumulate_raw(const DrawRow<E>& d, const RawSub<E>& r, int u, double apos,
                                               double aneg, const double* tab, BlockSums& b) {
    if constexpr (sizeof(typename E::T) == 2) {
        // bf16: four tokens at a time (more independent fp64 chains per wave;
        // the fp32 form would spill at this width)
#pragma unroll
        for (int k = 0; k < kSubTokens; k += 4) {
            float la = sub_logit<E>(r, k), lb = sub_logit<E>(r, k + 1);
            float lc = sub_logit<E>(r, k + 2), ld = sub_logit<E>(r, k + 3);
            if (k > 0) asm volatile("" : "+v"(la), "+v"(lb), "+v"(lc), "+v"(ld) : "v"(b.se));
            accumulate_token<E, kResidual>(d, la, kResidual ? sub_q<E>(r, k) : 0.0f, u * kSubTokens + k, apos,
                                           aneg, tab, b);
            accumulate_token<E, kResidual>(d, lb, kResidual ? sub_q<E>(r, k + 1) : 0.0f, u * kSubTokens + k + 1,
                                           apos, aneg, tab, b);
            accumulate_token<E, kResidual>(d, lc, kResidual ? sub_q<E>(r, k + 2) : 0.0f, u * kSubTokens + k + 2,
                                           apos, aneg, tab, b);
            accumulate_token<E, kResidual>(d, ld, kResidual ? sub_q<E>(r, k + 3) : 0.0f, u * kSubTokens + k + 3,
                                           apos, aneg, tab, b);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll
        for (int k = 0; k < kSubTokens; k += 2) {
            float la = sub_logit<E>(r, k), lb = sub_logit<E>(r, k + 1);
            if (k > 0) asm volatile("" : "+v"(la), "+v"(lb) : "v"(b.se));
            accumulate_token<E, kResidual>(d, la, kResidual ? sub_q<E>(r, k) : 0.0f, u * kSubTokens + k, apos,
                                           aneg, tab, b);
            accumulate_token<E, kResidual>(d, lb, kResidual ? sub_q<E>(r, k + 1) : 0.0f, u * kSubTokens + k + 1,
                                           apos, aneg, tab, b);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Wave totals of a block's sums, written to its record with device-scope
// stores (plus the inline marginal tokens).  Wave-uniform call.
template <typename E, bool kResidual>
__device__ __forceinline__ void store_record(const DrawRow<E>& d, long xb, BlockSums b, const double* tab,
                                             BlockRec* rec) {
    const int lane = threadIdx.x & 63;
    const double se = wave_sum(b.se);
    double ea = 0.0, qa = 0.0;
    int nmw = 0;
    if (kResidual) {
        ea = wave_sum(b.ea);
        qa = wave_sum(b.qa);
        if (__ballot(b.mmask != 0u) != 0ull) nmw = wave_sum_int(__popc(b.mmask));
    }
    if (lane == 0) {
        st_coherent(&rec->se, se);
        st_coherent(&rec->ea, ea);
        st_coherent(&rec->qa, qa);
        st_coherent(&rec->nm, nmw);
    }
    if (kResidual && nmw > 0 && nmw <= kMarginSlots)
        record_marginal<E>(d.lrow, d.qrow, d.c2, d.mc2, xb, b.mmask, tab, rec);
}

// Sums of one loaded block (any row layout).
template <typename E, bool kResidual>
__device__ __forceinline__ void block_record(const DrawRow<E>& d, const RawBlock<E>& r, long xb, int V, double apos,
                                             double aneg, const double* tab, BlockRec* rec) {
    BlockSums b;
#pragma unroll
    for (int u = 0; u < kSubBlocks; ++u) {
        // (a sub-block wholly past the row's end weighs nothing)
        if (xb + u * kSubElems >= V) continue;
        float l[kSubTokens], q[kSubTokens];
        decode_sub<E>(r.s[u], kResidual, l, q);
        accumulate_sub<E, kResidual>(d, l, q, u, apos, aneg, tab, b);
    }
    store_record<E, kResidual>(d, xb, b, tab, rec);
}

// Loads of this lane's tokens [x0, x0 + 8) of a block lying wholly inside a
// 16-byte aligned row (and q row).  Cache policy, as measured with the inputs
// rotating over more than the Infinity Cache holds: q rows with the default
// policy, logits non-temporal beside a q row and default-policy without one
// (B = 64, V = 151936: 44.2-44.4 us per step against 44.7-45.1 with every
// load default-policy and 44.9 with every load non-temporal; B = 256 ragged
// 98.4 against 99.4 and 100.3; point-mass q, logits only, 37.8 default-policy
// against 38.3 non-temporal).
template <typename E, bool kWithQ>
__device__ __forceinline__ void issue_sub_full(const DrawRow<E>& d, int x0, RawSub<E>& r) {
    const v4u* lp = reinterpret_cast<const v4u*>(d.lrow + x0);
#pragma unroll
    for (int h = 0; h < kSubTokens / E::kPerVec; ++h) r.l[h] = kWithQ ? __builtin_nontemporal_load(lp + h) : lp[h];
    if (kWithQ) {
        const v4u* qp = reinterpret_cast<const v4u*>(d.qrow + x0);
#pragma unroll
        for (int h = 0; h < kSubTokens / 4; ++h) r.q[h] = qp[h];
    }
}

// This lane's first token of sub-block u of the block starting at xb (32-bit:
// rows hold at most 2^19 tokens).
__device__ __forceinline__ int sub_first32(int xb, int u) {
    return xb + u * kSubElems + (threadIdx.x & 63) * kSubTokens;
}

// Wave totals of one streamed block, stored to its record; a block with inline
// marginal tokens is remembered (at most two per stream; further ones are left
// for the select to re-evaluate from their tokens) and captured after the
// stream has ended.
struct StreamCaps {
    int n = 0;                    // wave-uniform
    int j0 = 0, j1 = 0;           // blocks to capture
    uint32_t m0 = 0u, m1 = 0u;    // their marginal masks (per lane)
};

template <bool kResidual>
__device__ __forceinline__ void stream_finish(const BlockSums& b, int j, BlockRec* recs, StreamCaps& c) {
    const int lane = threadIdx.x & 63;
    const double se = wave_sum(b.se);
    double ea = 0.0, qa = 0.0;
    int nm = 0;
    if (kResidual) {
        ea = wave_sum(b.ea);
        qa = wave_sum(b.qa);
        if (__ballot(b.mmask != 0u) != 0ull) nm = wave_sum_int(__popc(b.mmask));
    }
    if (kResidual && nm > 0 && nm <= kMarginSlots) {
        // selects rather than branches, so the fields stay in registers
        const bool first = (c.n == 0), second = (c.n == 1);
        c.j0 = first ? j : c.j0;
        c.m0 = first ? b.mmask : c.m0;
        c.j1 = second ? j : c.j1;
        c.m1 = second ? b.mmask : c.m1;
        if (c.n >= 2) nm = kMarginSlots + 1;
        c.n = min(c.n + 1, 2);
    }
    if (lane == 0) {
        BlockRec* rec = &recs[j];
        st_coherent(&rec->se, se);
        st_coherent(&rec->ea, ea);
        st_coherent(&rec->qa, qa);
        st_coherent(&rec->nm, nm);
    }
}

// Blocks j and, if kN == 2, j2 of a whole-vector row, streamed as one sequence
// of sub-blocks (block j's four, then j2's) with kStreamDepth sub-blocks' loads
// in flight: a sub-block's registers are refilled with the one kStreamDepth
// further on as soon as its tokens are summed.  A wave thus asks for a few KB at
// a time, and the loads of all the waves meet the memory system interleaved: a
// wave that starts late is not queued behind whole blocks of earlier waves, and
// the tokens arrive spread over the stream instead of in per-wave bursts.
// Straight-line code (a loop around it spills; a call would leave the compiler
// unable to wait for one refill while the later ones stay in flight).
constexpr int kStreamDepth = 2;
template <typename E, bool kResidual, int kN>
__device__ __forceinline__ void stream_subs(const DrawRow<E>& d, BlockRec* recs, int j, int j2, double apos,
                                            double aneg, const double* tab, StreamCaps& c) {
    constexpr int K = kSubBlocks * kN;
    RawSub<E> slot[kStreamDepth];
#pragma unroll
    for (int k = 0; k < kStreamDepth && k < K; ++k)
        issue_sub_full<E, kResidual>(d, sub_first32((k < kSubBlocks ? j : j2) * kBlockElems, k % kSubBlocks), slot[k]);
    BlockSums b;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        accumulate_raw<E, kResidual>(d, slot[k % kStreamDepth], k % kSubBlocks, apos, aneg, tab, b);
        if (k + kStreamDepth < K) {
            const int kn = k + kStreamDepth;
            issue_sub_full<E, kResidual>(d, sub_first32((kn < kSubBlocks ? j : j2) * kBlockElems, kn % kSubBlocks),
                                         slot[k % kStreamDepth]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (k % kSubBlocks == kSubBlocks - 1) {
            stream_finish<kResidual>(b, k < kSubBlocks ? j : j2, recs, c);
            b = BlockSums();
        }
    }
}

// Blocks j and, if n == 2, j + jstride of a whole-vector row.
template <typename E, bool kResidual>
__device__ __forceinline__ void draw_blocks_upto2(const DrawRow<E>& d, int V, BlockRec* recs, int j, int jstride,
                                                  int n, double apos, double aneg, const double* tab,
                                                  StreamCaps& c) {
    if (n >= 2) stream_subs<E, kResidual, 2>(d, recs, j, j + jstride, apos, aneg, tab, c);
    else stream_subs<E, kResidual, 1>(d, recs, j, j, apos, aneg, tab, c);
}

template <typename E, bool kResidual>
__device__ __forceinline__ void capture_marginals(const DrawRow<E>& d, BlockRec* recs, const StreamCaps& c,
                                                  const double* tab) {
    if (kResidual && c.n > 0)
        record_marginal<E>(d.lrow, d.qrow, d.c2, d.mc2, (long)c.j0 * kBlockElems, c.m0, tab, &recs[c.j0]);
    if (kResidual && c.n > 1)
        record_marginal<E>(d.lrow, d.qrow, d.c2, d.mc2, (long)c.j1 * kBlockElems, c.m1, tab, &recs[c.j1]);
}

// Per-block sums of draw blocks jfirst, jfirst + jstride, ... < jend, written to
// recs.  In 16-byte aligned rows, blocks lying wholly inside the row are taken
// two at a time as one stream of sub-blocks (stream_subs; kUpTo2: the caller
// guarantees at most two blocks, and no loop is generated around them); the
// row's ragged last block, and every block of other rows, is taken on its own.
template <typename E, bool kResidual, bool kUpTo2>
__device__ __forceinline__ void draw_blocks_kind(const DrawRow<E>& d, int V, BlockRec* recs, int jfirst, int jstride,
                                                 int jend, const double* tab) {
    const double invZ32 = 1.0 / d.z32;
    const double apos = invZ32 * (1.0 - kSignMargin), aneg = invZ32 * (1.0 + kSignMargin);
    const bool fastrow = d.lalign && (!kResidual || d.qalign);
    const int jfull = V / kBlockElems;             // blocks wholly inside the row
    if constexpr (kUpTo2) {
        // this wave's blocks j1 = jfirst and j2 = jfirst + jstride (those below
        // jend).  The row's ragged last block jr = jfull, read in a round trip of
        // its own after the wave's stream, would otherwise end a wave that also
        // streams a full block: it trades places with the last block of the last
        // wave, which holds the fewest blocks
        int j1 = jfirst, j2 = jfirst + jstride;
        const int nb = (j1 < jend ? 1 : 0) + (j2 < jend ? 1 : 0);
        if (fastrow && jfull < jend && jfull >= jstride) {
            const int jr = jfull, wr = jr - jstride, xw = jstride - 1;
            const int X = xw + jstride < jend ? xw + jstride : xw;
            if (wr != xw && X != jr) {
                if (jfirst == wr) j2 = X;
                else if (jfirst == xw) {
                    if (X == xw) j1 = jr;
                    else j2 = jr;
                }
            }
        }
        const bool f1 = fastrow && nb >= 1 && j1 < jfull, f2 = fastrow && nb >= 2 && j2 < jfull;
        if (f1) {
            StreamCaps c;
            if (f2) stream_subs<E, kResidual, 2>(d, recs, j1, j2, apos, aneg, tab, c);
            else stream_subs<E, kResidual, 1>(d, recs, j1, j1, apos, aneg, tab, c);
            capture_marginals<E, kResidual>(d, recs, c, tab);
        }
        // the rest on their own (a ragged block, or a row that is not aligned)
        for (int t = 0; t < nb; ++t) {
            if (t == 0 ? f1 : f2) continue;
            const int j = t == 0 ? j1 : j2;
            RawBlock<E> r;
            const long xb = (long)j * kBlockElems;
            issue_block_any<E>(d, xb, V, kResidual, r);
            block_record<E, kResidual>(d, r, xb, V, apos, aneg, tab, &recs[j]);
        }
        return;
    }
    int jany = jfirst;                             // first block taken on its own
    if (fastrow) {
        const int jend_full = jend < jfull ? jend : jfull;
        StreamCaps c;
        int j = jfirst;
        {
            while (j < jend_full) {
                const int n = j + jstride < jend_full ? 2 : 1;
                draw_blocks_upto2<E, kResidual>(d, V, recs, j, jstride, n, apos, aneg, tab, c);
                j += n * jstride;
            }
        }
        capture_marginals<E, kResidual>(d, recs, c, tab);
        jany = j;
    }
    for (int j = jany; j < jend; j += jstride) {
        RawBlock<E> r;
        const long xb = (long)j * kBlockElems;
        issue_block_any<E>(d, xb, V, kResidual, r);
        block_record<E, kResidual>(d, r, xb, V, apos, aneg, tab, &recs[j]);
    }
}

// Split blocks: the four waves' sums of one block, met in LDS.
struct SplitShared {
    double se[kWaves], ea[kWaves], qa[kWaves];
    uint32_t mm[kWaves][64];     // every lane's marginal bits
};

// Split blocks (a call small enough for one workgroup per block in one
// resident round): wave u streams sub-block u of block j (element-wise where
// the row's alignment or end requires it), the four waves' sums meet in LDS and
// wave 0 stores the block's record; a wave then holds 512 tokens, not a whole
// block.  Uniform call.
template <typename E, bool kResidual>
__device__ __forceinline__ void draw_block_split_kind(const DrawRow<E>& d, int V, BlockRec* recs, int j,
                                                      const double* tab, SplitShared& ss) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const double invZ32 = 1.0 / d.z32;
    const double apos = invZ32 * (1.0 - kSignMargin), aneg = invZ32 * (1.0 + kSignMargin);
    const long xb = (long)j * kBlockElems;
    RawSub<E> r;
    issue_sub_any<E>(d, sub_first(xb, wv), V, kResidual, r);
    float l[kSubTokens], q[kSubTokens];
    decode_sub<E>(r, kResidual, l, q);
    BlockSums b;
    accumulate_sub<E, kResidual>(d, l, q, wv, apos, aneg, tab, b);
    const double se = wave_sum(b.se);
    const double ea = kResidual ? wave_sum(b.ea) : 0.0;
    const double qa = kResidual ? wave_sum(b.qa) : 0.0;
    if (lane == 0) {
        ss.se[wv] = se;
        ss.ea[wv] = ea;
        ss.qa[wv] = qa;
    }
    ss.mm[wv][lane] = b.mmask;
    __syncthreads();
    if (wv == 0) {
        // the block's totals on lane 0 (sub-block order), every lane's bits of
        // all four sub-blocks: store_record's wave sums then give the totals
        BlockSums t;
        t.se = lane == 0 ? ((ss.se[0] + ss.se[1]) + ss.se[2]) + ss.se[3] : 0.0;
        t.ea = lane == 0 ? ((ss.ea[0] + ss.ea[1]) + ss.ea[2]) + ss.ea[3] : 0.0;
        t.qa = lane == 0 ? ((ss.qa[0] + ss.qa[1]) + ss.qa[2]) + ss.qa[3] : 0.0;
        t.mmask = ss.mm[0][lane] | ss.mm[1][lane] | ss.mm[2][lane] | ss.mm[3][lane];
        store_record<E, kResidual>(d, xb, t, tab, &recs[j]);
    }
}

template <typename E>
__device__ __forceinline__ void draw_block_split(const DrawRow<E>& d, int V, BlockRec* recs, int j, const double* tab,
                                                 SplitShared& ss) {
    if (d.kind == kDrawResidual && !d.qlist) draw_block_split_kind<E, true>(d, V, recs, j, tab, ss);
    else draw_block_split_kind<E, false>(d, V, recs, j, tab, ss);
}

template <typename E, bool kUpTo2 = false>
__device__ __forceinline__ void draw_blocks(const DrawRow<E>& d, int V, BlockRec* recs, int jfirst, int jstride, int jend,
                            const double* tab) {
    if (d.kind == kDrawResidual && !d.qlist) draw_blocks_kind<E, true, kUpTo2>(d, V, recs, jfirst, jstride, jend, tab);
    else draw_blocks_kind<E, false, kUpTo2>(d, V, recs, jfirst, jstride, jend, tab);
}

// The select for one request, once all its draw blocks are recorded: the block
// holding the draw, then the token inside it.
//
// Block choice, by one wave (no LDS besides the exponential table; every lane
// gets the result).  Rebuilds the exact fp64 normaliser Z64 and every block's
// weight (e / Z64 - q summed over the clearly positive tokens plus the inline
// marginal ones; blocks with more marginal tokens than slots, or every block
// when the fp32-pass normaliser is off by more than half the margin, are
// re-evaluated from their tokens) and finds the block holding v * S by a scan
// over blocks (kSelPer consecutive blocks per lane).
struct SelBlock {
    int jsel;            // selected block
    double base;         // weight of the blocks before it
    double tsel;         // v * S
    double invZ64;
    bool res_w;          // token weights are residuals (else e)
    bool with_q;         // residual weights read a dense q row (else q = 0 off the list)
    bool fallback;       // rounding left no crossing: take the block's last positive token
    // listed q (sparse or point mass): lane s holds entry s; qmask: the entries
    // inside the selected block (wave-uniform)
    int qid;
    float qq;
    unsigned long long qmask;
};

template <typename E>
__device__ __forceinline__ SelBlock select_block(const DrawRow<E>& d, int V, int NB, const BlockRec* recs,
                                                 const double* tab, uint32_t* err, uint32_t* err_host) {
    const int lane = threadIdx.x & 63;
    const bool residual = (d.kind == kDrawResidual);
    // every field of this lane's records in one round of loads
    double se_t[kSelPer], ea_t[kSelPer], qa_t[kSelPer];
    int nm_t[kSelPer];
#pragma unroll
    for (int r = 0; r < kSelPer; ++r) {
        const int j = lane * kSelPer + r;
        const bool in = j < NB;
        const BlockRec* rc = &recs[in ? j : 0];
        se_t[r] = in ? ld_coherent(&rc->se) : 0.0;
        ea_t[r] = qa_t[r] = 0.0;
        nm_t[r] = 0;
        if (residual && !d.qlist && in) {
            ea_t[r] = ld_coherent(&rc->ea);
            qa_t[r] = ld_coherent(&rc->qa);
            nm_t[r] = ld_coherent(&rc->nm);
        }
    }
    double zpart = 0.0;
#pragma unroll
    for (int r = 0; r < kSelPer; ++r) zpart += se_t[r];
    const double Z64 = wave_sum(zpart);
    const double invZ64 = 1.0 / Z64;
    int kind = d.kind;
    double wt[kSelPer];
    int qid = -1;
    float qq = 0.0f;
    bool qvalid = false;
    if (residual && d.qlist) {
        // q is zero except at the listed tokens: block weights are the blocks' p
        // mass less min(p, q) of the listed tokens they hold (p - (p - q)_+)
        if (lane < d.nq) {
            qid = d.sid[lane];
            qq = d.sq ? d.sq[lane] : 1.0f;
        }
        qvalid = qid >= 0 && qid < V;
        if (lane < d.nq && !qvalid && qid != -1) flag_error(err, err_host, kErrTopk);
        double cs = 0.0;
        if (qvalid) cs = fmin(draw_e<E>(d, E::load1(d.lrow, qid), tab) * invZ64, static_cast<double>(qq));
        const int qblk = qvalid ? qid / kBlockElems : -1;
#pragma unroll
        for (int r = 0; r < kSelPer; ++r) wt[r] = se_t[r] * invZ64;
        for (int s = 0; s < d.nq; ++s) {
            const int js = rdlane(qblk, s);
            if (js < 0) continue;
            const double c = rdlane(cs, s);
#pragma unroll
            for (int r = 0; r < kSelPer; ++r)
                if (lane * kSelPer + r == js) wt[r] -= c;
        }
    } else if (residual) {
        const bool full = !(fabs(Z64 - d.z32) <= 0.5 * kSignMargin * Z64);
#pragma unroll
        for (int r = 0; r < kSelPer; ++r) wt[r] = ea_t[r] * invZ64 - qa_t[r];
        // blocks with inline marginal tokens (a slot is only meaningful when the
        // block recorded it): one more round of loads, only when there are any
        bool any_slots = false;
#pragma unroll
        for (int r = 0; r < kSelPer; ++r) any_slots |= (nm_t[r] > 0 && nm_t[r] <= kMarginSlots);
        if (__ballot(any_slots) != 0ull) {
#pragma unroll
            for (int r = 0; r < kSelPer; ++r) {
                const int j = lane * kSelPer + r;
                if (j < NB && nm_t[r] > 0 && nm_t[r] <= kMarginSlots) {
                    const BlockRec* rc = &recs[j];
                    wt[r] += fmax(ld_coherent(&rc->me[0]) * invZ64 - static_cast<double>(ld_coherent(&rc->mq[0])), 0.0);
                    if (nm_t[r] > 1)
                        wt[r] += fmax(ld_coherent(&rc->me[1]) * invZ64 - static_cast<double>(ld_coherent(&rc->mq[1])), 0.0);
                }
            }
        }
        // rare: blocks re-evaluated from their tokens, one at a time by the wave,
        // a sub-block per round trip.  One copy of the body, not unrolled: the
        // select runs once per request, on code the stream has usually pushed
        // out of the instruction cache, and every line of code it passes costs
        unsigned long long needs[kSelPer];
#pragma unroll
        for (int r = 0; r < kSelPer; ++r)
            needs[r] = __ballot(lane * kSelPer + r < NB && (full || nm_t[r] > kMarginSlots));
        unsigned long long anyneed = 0ull;
#pragma unroll
        for (int r = 0; r < kSelPer; ++r) anyneed |= needs[r];
        if (anyneed != 0ull) {
#pragma unroll 1
            for (int r = 0; r < kSelPer; ++r) {
                unsigned long long need = needs[0];
#pragma unroll
                for (int rr = 1; rr < kSelPer; ++rr)
                    if (rr == r) need = needs[rr];
                while (need != 0ull) {
                    const int L = __ffsll(static_cast<long long>(need)) - 1;
                    need &= need - 1ull;
                    const long xb = (long)(L * kSelPer + r) * kBlockElems;
                    double w = 0.0;
#pragma unroll 1
                    for (int u = 0; u < kSubBlocks; ++u) {
                        RawSub<E> raw;
                        issue_sub_any<E>(d, sub_first(xb, u), V, true, raw);
                        float l[kSubTokens], q[kSubTokens];
                        decode_sub<E>(raw, true, l, q);
#pragma unroll
                        for (int k = 0; k < kSubTokens; ++k)
                            w += fmax(draw_e<E>(d, l[k], tab) * invZ64 - static_cast<double>(q[k]), 0.0);
                    }
                    w = wave_sum(w);
#pragma unroll
                    for (int rr = 0; rr < kSelPer; ++rr)
                        if (rr == r && lane == L) wt[rr] = w;
                }
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < kSelPer; ++r) wt[r] = se_t[r];
    }
    // ---- block scan
    double own = 0.0;
#pragma unroll
    for (int r = 0; r < kSelPer; ++r) own += wt[r];
    double incl = wave_inclusive_scan(own);
    double Stot = rdlane(incl, 63);
    if (residual && !(Stot > 0.0)) {
        // residual lost to rounding: draw from p itself
        kind = kDrawDegenerate;
        own = 0.0;
#pragma unroll
        for (int r = 0; r < kSelPer; ++r) { wt[r] = se_t[r]; own += wt[r]; }
        incl = wave_inclusive_scan(own);
        Stot = rdlane(incl, 63);
    }
    const double tsel = static_cast<double>(d.v) * Stot;
    // this lane's first block whose inclusive sum passes tsel, and its last block
    // of positive weight, each with the sum before it
    int cand = -1, lastpos = -1;
    double cand_before = 0.0, last_before = 0.0;
    {
        double run = incl - own;
#pragma unroll
        for (int r = 0; r < kSelPer; ++r) {
            const int j = lane * kSelPer + r;
            const double before = run;
            run += wt[r];
            if (j < NB && wt[r] > 0.0) { lastpos = j; last_before = before; }
            if (j < NB && cand < 0 && run > tsel) { cand = j; cand_before = before; }
        }
    }
    const unsigned long long cm = __ballot(cand >= 0), lm = __ballot(lastpos >= 0);
    int jsel;
    double base;
    bool block_fallback = false;
    if (cm != 0ull) {
        const int L = __ffsll(static_cast<long long>(cm)) - 1;
        jsel = rdlane(cand, L);
        base = rdlane(cand_before, L);
    } else if (lm != 0ull) {            // rounding left no block above v * S: the last positive one
        const int L = 63 - __clzll(static_cast<long long>(lm));
        jsel = rdlane(lastpos, L);
        base = rdlane(last_before, L);
        block_fallback = true;
    } else {                            // no positive finite weight (non-finite logits)
        jsel = 0;
        base = 0.0;
        block_fallback = true;
        if (lane == 0) flag_error(err, err_host, kErrNonFinite);
    }
    SelBlock sb;
    sb.jsel = jsel;
    sb.base = base;
    sb.tsel = tsel;
    sb.invZ64 = invZ64;
    sb.res_w = (kind == kDrawResidual);
    sb.with_q = sb.res_w && !d.qlist;
    sb.fallback = block_fallback;
    sb.qid = qid;
    sb.qq = qq;
    sb.qmask = sb.res_w ? __ballot(qvalid && qid / kBlockElems == jsel) : 0ull;
    return sb;
}

// Token weights of one lane's 8 tokens of sub-block u of the selected block, and
// their sum (tokens past the row's end weigh nothing).
template <typename E>
__device__ __forceinline__ double sub_weights(const DrawRow<E>& d, const RawSub<E>& raw, long x0, int V,
                                              const SelBlock& sb, const double* tab, double* w) {
    float l[kSubTokens], q[kSubTokens];
    decode_sub<E>(raw, sb.with_q, l, q);
#pragma unroll
    for (int k = 0; k < kSubTokens; ++k) {
        const double e = draw_e<E>(d, l[k], tab);
        w[k] = sb.res_w ? fmax(e * sb.invZ64 - static_cast<double>(q[k]), 0.0) : e;
        if (x0 + k >= V) w[k] = 0.0;
        if (k & 1) __builtin_amdgcn_sched_barrier(0);
    }
    // listed q entries among this lane's tokens (q was taken as 0 above)
    unsigned long long m = sb.qmask;
    while (m != 0ull) {
        const int s = __ffsll(static_cast<long long>(m)) - 1;
        m &= m - 1ull;
        const int xi = rdlane(sb.qid, s);
        const double qv = static_cast<double>(rdlane(sb.qq, s));
#pragma unroll
        for (int k = 0; k < kSubTokens; ++k)
            if (x0 + k == xi) w[k] = fmax(w[k] - qv, 0.0);
    }
    double tsum = 0.0;
#pragma unroll
    for (int k = 0; k < kSubTokens; ++k) tsum += w[k];
    return tsum;
}

// Walks one lane's weights in token order from run (the sum before its first
// token): the first token whose running sum passes tsel, and the last token of
// positive weight.
__device__ __forceinline__ void sub_find(const double* w, long x0, double run, const SelBlock& sb, int& ycand,
                                         int& ylast) {
#pragma unroll
    for (int k = 0; k < kSubTokens; ++k) {
        run += w[k];
        const int x = static_cast<int>(x0) + k;
        if (w[k] > 0.0) ylast = x;
        if (!sb.fallback && ycand == 0x7fffffff && run > sb.tsel) ycand = x;
    }
}

// The token, given the first crossing and the last positive token found.
__device__ __forceinline__ int select_token(int ycand, int ylast, int V, int jsel) {
    int y = ycand;
    if (y == 0x7fffffff) y = ylast;
    if (y < 0) y = min(V - 1, jsel * kBlockElems + kBlockElems - 1);
    return y;
}

// The same select by a whole workgroup: every wave makes the (identical) block
// choice, then wave u scans sub-block u, so the block is loaded in one round;
// the sub-block sums and each wave's finds meet in LDS.  Every thread returns
// the token.  Uniform call.
static_assert(kSubBlocks == kWaves, "one sub-block per wave");
struct SelShared {
    double tot[kWaves];
    int yc[kWaves], yl[kWaves];
    double zs[kWaves];       // (single-block draws) wave sums of e
};

template <typename E>
__device__ __forceinline__ int draw_select_wg(const DrawRow<E>& d, int V, int NB, const BlockRec* recs,
                                              const double* tab, uint32_t* err, uint32_t* err_host,
                                              SelShared& ss) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const SelBlock sb = select_block<E>(d, V, NB, recs, tab, err, err_host);
    const long x0 = sub_first((long)sb.jsel * kBlockElems, wv);
    RawSub<E> raw;
    issue_sub_any<E>(d, x0, V, sb.with_q, raw);
    double w[kSubTokens];
    const double tsum = sub_weights<E>(d, raw, x0, V, sb, tab, w);
    const double ti = wave_inclusive_scan(tsum);
    if (lane == 63) ss.tot[wv] = ti;
    __syncthreads();
    // the sums before this sub-block, added in sub-block order
    double run_base = sb.base;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) run_base += (u < wv) ? ss.tot[u] : 0.0;
    int ycand = 0x7fffffff, ylast = -1;
    sub_find(w, x0, run_base + (ti - tsum), sb, ycand, ylast);
    ycand = wave_min_int(ycand);
    ylast = wave_max_int(ylast);
    if (lane == 0) { ss.yc[wv] = ycand; ss.yl[wv] = ylast; }
    __syncthreads();
    int yc = ss.yc[0], yl = ss.yl[0];
#pragma unroll
    for (int u = 1; u < kWaves; ++u) { yc = min(yc, ss.yc[u]); yl = max(yl, ss.yl[u]); }
    return select_token(yc, yl, V, sb.jsel);
}

// The whole draw of a row that is a single block (V <= 2048), by the request's
// only workgroup: wave u loads sub-block u once and keeps it; Z64 (every
// token's e, wave sums met in LDS in wave order), the token weights with the
// exact normaliser, their sum S and the token holding v * S all come from
// those registers.  No block record, no marginal tokens, no second read.
// Every thread returns the token.  Uniform call.
template <typename E>
__device__ __forceinline__ int draw_single_block(const DrawRow<E>& d, int V, const double* tab, uint32_t* err,
                                                 uint32_t* err_host, SelShared& ss) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool residual = (d.kind == kDrawResidual);
    SelBlock sb;
    sb.jsel = 0;
    sb.base = 0.0;
    sb.fallback = false;
    sb.qid = -1;
    sb.qq = 0.0f;
    if (residual && d.qlist && lane < d.nq) {
        sb.qid = d.sid[lane];
        sb.qq = d.sq ? d.sq[lane] : 1.0f;
    }
    const long x0 = sub_first(0, wv);
    RawSub<E> raw;
    issue_sub_any<E>(d, x0, V, residual && !d.qlist, raw);
    const bool qvalid = sb.qid >= 0 && sb.qid < V;
    if (wv == 0 && lane < d.nq && !qvalid && sb.qid != -1) flag_error(err, err_host, kErrTopk);
    double se = 0.0;
#pragma unroll
    for (int k = 0; k < kSubTokens; ++k) {
        if (x0 + k < V) se += draw_e<E>(d, sub_logit<E>(raw, k), tab);
        if (k & 1) __builtin_amdgcn_sched_barrier(0);
    }
    const double zw = wave_sum(se);
    if (lane == 0) ss.zs[wv] = zw;
    __syncthreads();
    sb.invZ64 = 1.0 / (((ss.zs[0] + ss.zs[1]) + ss.zs[2]) + ss.zs[3]);
    sb.res_w = residual;
    sb.with_q = residual && !d.qlist;
    // every listed token lies in the one block
    sb.qmask = residual ? __ballot(qvalid) : 0ull;
    double w[kSubTokens];
    double tsum = sub_weights<E>(d, raw, x0, V, sb, tab, w);
    double ti = wave_inclusive_scan(tsum);
    if (lane == 63) ss.tot[wv] = ti;
    __syncthreads();
    double Stot = ((ss.tot[0] + ss.tot[1]) + ss.tot[2]) + ss.tot[3];
    if (residual && !(Stot > 0.0)) {
        // residual lost to rounding: draw from p itself
        sb.res_w = false;
        sb.with_q = false;
        sb.qmask = 0ull;
        __syncthreads();                 // every thread has read the first sums
        tsum = sub_weights<E>(d, raw, x0, V, sb, tab, w);
        ti = wave_inclusive_scan(tsum);
        if (lane == 63) ss.tot[wv] = ti;
        __syncthreads();
        Stot = ((ss.tot[0] + ss.tot[1]) + ss.tot[2]) + ss.tot[3];
    }
    if (!(Stot > 0.0) && tid == 0) flag_error(err, err_host, kErrNonFinite);
    sb.tsel = static_cast<double>(d.v) * Stot;
    double run_base = 0.0;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) run_base += (u < wv) ? ss.tot[u] : 0.0;
    int ycand = 0x7fffffff, ylast = -1;
    sub_find(w, x0, run_base + (ti - tsum), sb, ycand, ylast);
    ycand = wave_min_int(ycand);
    ylast = wave_max_int(ylast);
    if (lane == 0) { ss.yc[wv] = ycand; ss.yl[wv] = ylast; }
    __syncthreads();
    int yc = ss.yc[0], yl = ss.yl[0];
#pragma unroll
    for (int u = 1; u < kWaves; ++u) { yc = min(yc, ss.yc[u]); yl = max(yl, ss.yl[u]); }
    return select_token(yc, yl, V, 0);
}

template <typename E>
__device__ __forceinline__ void init_draw_row(DrawRow<E>& d, const Params& P, int kind, int row, int drow,
                                              int pos, float v, float m, double z32, float T) {
    d.kind = kind;
    d.pos = pos;
    d.v = v;
    d.m = static_cast<double>(m);
    d.c2 = kExp2Scale * (kLog2e / static_cast<double>(T));
    d.mc2 = d.m * d.c2;
    d.z32 = z32;
    d.lrow = static_cast<const typename E::T*>(P.logits) + (size_t)row * P.vocab;
    d.qlist = (kind == kDrawResidual) && P.qmode != kQDense;
    d.qrow = (kind == kDrawResidual && !d.qlist) ? P.q + (size_t)drow * P.vocab : nullptr;
    d.lalign = (reinterpret_cast<uintptr_t>(d.lrow) & 15u) == 0;
    d.qalign = (reinterpret_cast<uintptr_t>(d.qrow) & 15u) == 0;
    d.nq = 0;
    d.sid = nullptr;
    d.sq = nullptr;
    if (d.qlist && P.qmode == kQSparse) {
        d.nq = P.topk;
        d.sid = P.topk_ids + (size_t)drow * P.topk;
        d.sq = P.topk_probs + (size_t)drow * P.topk;
    } else if (d.qlist) {
        d.nq = 1;
        d.sid = P.ids + drow;
    }
}

static_assert(kExp2TableSize % kThreads == 0, "whole table entries per draw thread");
constexpr int kTabPerThread = kExp2TableSize / kThreads;
struct DrawShared {
    double tab[kExp2TableSize];
    SelShared sel;
    SplitShared split;
    int flag;
};

// ----------------------------------------------------------------- resolve in the draw kernel
// After the stream-only rows kernel, every draw workgroup of request b rebuilds
// the request's row statistics from the stored pieces, runs the accept tests
// and finds the first rejection itself (a few hundred bytes of loads and a
// handful of fp64 exponentials: cheaper than a hand-off between workgroups);
// the request's workgroup 0 writes the outputs, except the drawn token, which
// the select writes.
constexpr int kMaxReqRows = 129;          // gamma_b + 1 rows of one request at most
constexpr int kResolveChunk = 8;          // pieces a thread loads in one round

struct ResolveShared {
    float rm[kMaxReqRows];       // row max (sampled) / argmax value (greedy)
    double rz[kMaxReqRows];      // row normaliser
    int rej[kMaxReqRows];        // draft i rejected
    uint32_t bad[kMaxReqRows];   // contract violations found on row i (kErr* bits)
};

// Outputs of a request that breaks the device-side contract: every token and
// num_accepted are -1 (written by the request's writer workgroup only).
__device__ __forceinline__ void write_violation(const Params& P, int b) {
    const int tid = threadIdx.x;
    for (int j = tid; j <= P.gamma; j += kThreads) P.out_tokens[(size_t)b * (P.gamma + 1) + j] = -1;
    if (tid == 0) P.out_num[b] = -1;
}

// Uniform call.  Returns request b's draw task (kDrawNone: greedy, nothing to
// draw, or a request that breaks the device-side contract); `writer`
// workgroups store the outputs, counters and diagnostics.  Thread i owns row i
// of the request: it loads the row's pieces and its draft's id, logit, q and
// uniform in one round, merges the pieces and runs the accept test, so that a
// single barrier publishes the rows' results.  A request is a contract
// violation when its offsets are inconsistent, a draft id lies outside
// [0, vocab), its sparse q breaks the entry rules, or one of its sampled rows
// has no positive finite normaliser (no finite logit, or NaN logits); its
// outputs are then all -1, the bits are flagged, and it is not counted.
template <typename E>
__device__ __forceinline__ DrawTask resolve_request(const Params& P, int b, bool writer, float T, ResolveShared& rs,
                                                   double* tab, const double* tv) {
    const int tid = threadIdx.x;
    const int G = P.gamma;
    DrawTask tk;
    tk.kind = kDrawNone;
    tk.row = tk.drow = tk.pos = 0;
    tk.v = tk.m = 0.0f;
    tk.z32 = 0.0;
    int o0, o1;
    if (P.offsets) {
        o0 = P.offsets[b];
        o1 = P.offsets[b + 1];
    } else {
        o0 = b * G;
        o1 = o0 + G;
    }
    const int gb = o1 - o0;
    if (!(o0 >= 0 && o1 <= P.total_draft && gb >= 0 && gb <= G && gb < kMaxReqRows)) {
        if (writer) {
            write_violation(P, b);
            if (tid == 0) flag_error(P.err, P.err_host, kErrOffsets);
        }
        return tk;
    }
    const int t0 = o0 + b;
    const bool greedy = !(T > 0.0f);
    // 1024 times the pieces' scale log2(e) / T as the rows kernel rounded it
    // (exact), and 1024 log2(e) / T for the accept ratio: exponentials by the
    // same table-based exp2 as the draw weights
    const double cpz = greedy ? 0.0 : kExp2Scale * static_cast<double>(static_cast<float>(kLog2e / static_cast<double>(T)));
    const double c2 = greedy ? 0.0 : kExp2Scale * (kLog2e / static_cast<double>(T));
    float v_res = P.uniforms[(size_t)b * (G + 2) + G];
    float v_bonus = P.uniforms[(size_t)b * (G + 2) + G + 1];
    const bool owner = tid <= gb;
    float M = -INFINITY;          // row max, or the argmax value
    int g = 0x7fffffff;           // argmax
    double Z = 0.0;
    int xid = -1;
    bool rej = false;
    double r = 0.0;
    int xs = -1, np = 0;
    float lx = 0.0f, qx = 0.0f, u = 0.0f;
    const Piece* pp = nullptr;
    float mm[kResolveChunk], mm2[kResolveChunk];
    int gg[kResolveChunk], gg2[kResolveChunk];
    double zz[kResolveChunk], zz2[kResolveChunk];
    // rows of more than kResolveChunk pieces: the second round of slots is
    // loaded with the first (the geometry's bound, not the row's count, decides)
    const bool two = P.max_pieces > kResolveChunk;
    if (owner) {
        // stored by the rows kernel: the launch boundary orders those stores
        // before these plain loads.  The row's first kResolveChunk piece slots
        // are loaded together with its piece count (slots past the count hold
        // stale values and are masked once it is in), so that no load waits for
        // another or for the temperature.
        // (the bonus row's drafted-token fields and uniform slot are loaded too
        // and left unused: no branch, so no copy that waits for them)
        const int t = t0 + tid;
        const RowStat* rp = &P.rows[t];
        np = rp->np;
        xs = rp->x;
        lx = rp->lx;
        qx = rp->qx;
        u = P.uniforms[(size_t)b * (G + 2) + tid];
        if (tid < gb) xid = P.ids[o0 + tid];
        pp = &P.parts[(size_t)t * kMaxPieces];
#pragma unroll
        for (int q = 0; q < kResolveChunk; ++q) {
            mm[q] = pp[q].m;
            gg[q] = pp[q].g;
            zz[q] = pp[q].z;
        }
        if (two) {
#pragma unroll
            for (int q = 0; q < kResolveChunk; ++q) {
                mm2[q] = pp[kResolveChunk + q].m;
                gg2[q] = pp[kResolveChunk + q].g;
                zz2[q] = pp[kResolveChunk + q].z;
            }
        }
    }
    // the exponential table (tv: this thread's entries, loaded by the caller
    // before everything above) into LDS only now, so that its wait does not
    // hold back the loads above; the barrier publishes it, and the loads are
    // complete after it
#pragma unroll
    for (int j = 0; j < kTabPerThread; ++j) tab[tid + j * kThreads] = tv[j];
    __syncthreads();
    // the draw's uniforms taken into registers here, with the other loads: their
    // first use comes after the writer's output stores, and a wait there would
    // wait for those stores too; the drafted token's logit, q and uniform too,
    // so that their conversions are not hoisted above the piece loads (which
    // would then wait for them)
    asm volatile("" : "+v"(v_res), "+v"(v_bonus), "+v"(lx), "+v"(qx), "+v"(u));
    if (owner) {
        np = min(max(np, 0), kMaxPieces);
#pragma unroll
        for (int q = 0; q < kResolveChunk; ++q) {
            if (q >= np) {
                mm[q] = -INFINITY;
                gg[q] = 0x7fffffff;
                zz[q] = 0.0;
            }
        }
        for (int p0 = 0; p0 < np; p0 += kResolveChunk) {
            if (p0 == kResolveChunk && two) {
#pragma unroll
                for (int q = 0; q < kResolveChunk; ++q) {
                    const bool in = p0 + q < np;
                    mm[q] = in ? mm2[q] : -INFINITY;
                    gg[q] = in ? gg2[q] : 0x7fffffff;
                    zz[q] = in ? zz2[q] : 0.0;
                }
            } else if (p0 > 0) {
#pragma unroll
                for (int q = 0; q < kResolveChunk; ++q) {
                    const bool in = p0 + q < np;
                    mm[q] = in ? pp[p0 + q].m : -INFINITY;
                    gg[q] = in ? pp[p0 + q].g : 0x7fffffff;
                    zz[q] = in ? pp[p0 + q].z : 0.0;
                }
            }
            if (!greedy) {
                // the pieces' sums rescaled to the row max, in piece order
                float Mc = M;
#pragma unroll
                for (int q = 0; q < kResolveChunk; ++q) Mc = fmaxf(Mc, mm[q]);
                if (Mc > M && M > -INFINITY)
                    Z *= exp2_tab((static_cast<double>(M) - static_cast<double>(Mc)) * cpz, tab);
                M = Mc;
                // every slot's factor first (one round of table reads); an empty
                // slot (max -inf, sum 0) adds 0, its factor being 0
                double f[kResolveChunk];
#pragma unroll
                for (int q = 0; q < kResolveChunk; ++q)
                    f[q] = exp2_tab((static_cast<double>(mm[q]) - static_cast<double>(M)) * cpz, tab);
#pragma unroll
                for (int q = 0; q < kResolveChunk; ++q) Z += zz[q] * f[q];
            } else {
#pragma unroll
                for (int q = 0; q < kResolveChunk; ++q) argmax_merge(M, g, mm[q], gg[q]);
            }
        }
        // accept test (page section 5.2: q floored at 1e-10, strict comparison);
        // p(x) by the draw weights' own expression
        uint32_t bad = 0u;
        if (tid < gb) {
            bool acc;
            if (xid < 0 || xid >= P.vocab) bad |= kErrDraftId;
            if (greedy) {
                acc = (xid == g);
            } else {
                if (xs == -2) bad |= kErrTopk;
                const double px = exp2_tab(fma(static_cast<double>(lx), c2, -(static_cast<double>(M) * c2)), tab) / Z;
                r = px / fmax(static_cast<double>(qx), kQFloor);
                acc = (xs >= 0) && (static_cast<double>(u) < fmin(1.0, r));
            }
            rej = !acc;
        }
        if (!greedy && !(Z > 0.0 && Z < INFINITY && fabsf(M) < INFINITY)) bad |= kErrNonFinite;
        rs.rm[tid] = M;
        rs.rz[tid] = Z;
        rs.rej[tid] = rej ? 1 : 0;
        rs.bad[tid] = bad;
    }
    __syncthreads();
    // contract violations anywhere in the request (every wave finds the same):
    // a lane per row, then the bits themselves only when there are any
    const int lane = tid & 63;
    uint32_t badl = 0u;
    for (int j = lane; j <= gb; j += 64) badl |= rs.bad[j];
    if (__ballot(badl != 0u) != 0ull) {
        uint32_t badq = 0u;
        for (int j = 0; j <= gb; ++j) badq |= rs.bad[j];
        if (writer) {
            write_violation(P, b);
            if (tid == 0) flag_error(P.err, P.err_host, badq);
        }
        return tk;
    }
    // k = the first rejected draft (every wave finds the same)
    int k = gb;
    for (int base = 0; base < gb; base += 64) {
        const unsigned long long m = __ballot(base + lane < gb && rs.rej[base + lane] != 0);
        if (m != 0ull) {
            k = base + __ffsll(static_cast<long long>(m)) - 1;
            break;
        }
    }
    if (writer) {
        if (owner) {
            if (P.diag_m) P.diag_m[t0 + tid] = M;
            if (P.diag_z) P.diag_z[t0 + tid] = greedy ? 0.0 : Z;
            if (tid < gb && P.diag_r) P.diag_r[o0 + tid] = greedy ? __uint_as_float(0x7fc00000u) : static_cast<float>(r);
        }
        if (tid <= G) {
            int tok = -1;
            if (tid < k) tok = xid;
            else if (tid == k && greedy) tok = g;
            // the drawn token's slot is the select's (another workgroup of this launch)
            if (!(tid == k && !greedy)) P.out_tokens[(size_t)b * (G + 1) + tid] = tok;
        }
        if (tid == 0) P.out_num[b] = k;
        if (P.stats) {
            uint32_t* S = P.stats;
            if (tid == 0) {
                count_add(&S[0], 1u);
                count_add(&S[1], static_cast<uint32_t>(gb));
                count_add(&S[2], static_cast<uint32_t>(k));
                if (k == gb) count_add(&S[3], 1u);
                count_add(&S[4 + k], 1u);
            }
            if (tid < gb && tid <= k) count_add(&S[5 + G + tid], 1u);
            if (tid < k) count_add(&S[5 + 2 * G + tid], 1u);
        }
    }
    if (greedy) return tk;
    tk.kind = k < gb ? kDrawResidual : kDrawBonus;
    tk.row = t0 + k;
    tk.drow = o0 + k;
    tk.pos = k;
    tk.v = k < gb ? v_res : v_bonus;
    tk.m = rs.rm[k];
    tk.z32 = rs.rz[k];
    return tk;
}

// kLoop: waves may hold more than two blocks (taken two at a time in a loop;
// such grids hold at most three workgroups per CU, so the register budget is
// that of three); otherwise the grid gives every wave at most two blocks
// (checked by the host).  The rows kernel only streamed: every workgroup first
// resolves its request.
template <typename E, bool kLoop, bool kSplit = false>
__global__ __launch_bounds__(kThreads, kLoop ? 3 : 4) void draw_kernel(Params P) {
    __shared__ DrawShared sh;
    __shared__ ResolveShared rsh;

    const int tid = threadIdx.x;
    const int C = P.draw_wgs;
    // a grid that is resident in one round is dispatched piece-index-major, so
    // that the workgroups holding the most blocks (low c) start first and the
    // lightest last (a CU serves its older workgroups first); a larger grid is
    // request-major, so that early requests finish while later ones wait for slots
    const int b = P.draw_cmajor ? static_cast<int>(blockIdx.x % P.batch) : static_cast<int>(blockIdx.x / C);
    const int c = P.draw_cmajor ? static_cast<int>(blockIdx.x / P.batch) : static_cast<int>(blockIdx.x - b * C);
    const int NB = P.nblocks;

    // the request's inputs, the temperature and the exponential table in one
    // round of loads (the resolve stores the table to LDS)
    double tv[kTabPerThread];
#pragma unroll
    for (int j = 0; j < kTabPerThread; ++j) tv[j] = kExp2Table[tid + j * kThreads];
    const float T = P.temperature[b];
    const DrawTask tk = resolve_request<E>(P, b, c == 0, T, rsh, sh.tab, tv);
    if (tk.kind == kDrawNone) return;
    const bool residual = (tk.kind == kDrawResidual);
    if (tk.row < 0 || tk.row >= P.total_draft + P.batch || tk.pos < 0 || tk.pos > P.gamma ||
        (residual && (tk.drow < 0 || tk.drow >= P.total_draft)))
        return;                                    // only reachable with inconsistent offsets
    DrawRow<E> d;
    init_draw_row<E>(d, P, tk.kind, tk.row, tk.drow, tk.pos, tk.v, tk.m, tk.z32, T);
    __syncthreads();
    if constexpr (kSplit) {
        if (NB == 1) {             // (then this is the request's only workgroup)
            const int y = draw_single_block<E>(d, P.vocab, sh.tab, P.err, P.err_host, sh.sel);
            if (tid == 0) P.out_tokens[(size_t)b * (P.gamma + 1) + tk.pos] = y;
            return;
        }
    }
    BlockRec* recs = P.recs + (size_t)b * NB;
    if constexpr (kSplit) draw_block_split<E>(d, P.vocab, recs, c, sh.tab, sh.split);
    else draw_blocks<E, !kLoop>(d, P.vocab, recs, c * kWaves + (tid >> 6), C * kWaves, NB, sh.tab);
    wait_stores();                 // every wave's record stores complete before the arrival
    __syncthreads();
    if (C > 1) {                   // (a request's only workgroup selects without arriving)
        if (tid == 0) sh.flag = (arrive(&P.draw_cnt[b]) == static_cast<uint32_t>(C - 1));
        __syncthreads();
        if (!sh.flag) return;
        if (tid == 0) reset_counter(&P.draw_cnt[b]);
    }
    const int y = draw_select_wg<E>(d, P.vocab, NB, recs, sh.tab, P.err, P.err_host, sh.sel);
    if (tid == 0) {
        P.out_tokens[(size_t)b * (P.gamma + 1) + tk.pos] = y;
    }
}

}  // namespace sv
