// One-launch verify step (the fast path for 16-byte aligned rows, gamma <= 30).
//
// Method: the spec-decoding page at dpshk.com/news/5598276, sections 3.1-3.2,
// 5.2-5.3 and 8 (see sv_device.h).  This file changes only how the same work
// is ordered on the chip, using the page's own observation (section 3.1, step
// 3) that verification stops at the first rejection: the draw of a request
// depends only on its rows up to that position.
//
// A persistent, cooperatively launched grid (all workgroups resident) runs:
//
//   row pieces  Every target row is cut into P equal pieces.  Pieces are taken
//               in position-major order (position 0 of every request, then
//               position 1, ...), workgroup w taking items w, w + grid, ...
//               A piece yields (max, fp32-exponential sum) or (max, argmax).
//               The last piece of a row merges the row and makes its accept
//               decision; decisions are OR-ed into a per-request word by CAS.
//               The update that makes a request decidable (first rejection
//               known, or every draft accepted and the bonus row done)
//               resolves it: outputs, then the draw parameters, then one
//               64-bit publication word tagged with the call's epoch.  The
//               update that completes the request's rows clears the word for
//               the next call.
//   deferral    A piece of a request already resolved at an earlier position
//               is not needed for the outputs (only for per-row statistics);
//               the workgroup sets it aside and streams it after its other
//               pieces, so the end of the step is non-critical streaming that
//               covers the latency of the last draws.
//   draws       Request b's draw row is cut into C chunks of 512-token blocks;
//               chunk b*C + c belongs to workgroup (b*C + c) mod grid.  Between
//               pieces a workgroup takes whichever of its chunks are published;
//               at the end it waits (bounded) for the rest.  The last chunk of
//               a request runs the select.
//
// The only waits are for publications, which are made by workgroups that
// never wait for anything but their own loads, so the grid always drains.
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kSpinLimit = 1 << 20;      // bounded wait for a publication (about a second)
constexpr int kMaxGammaFused = 30;       // decided bits 0..30 of the per-request word
constexpr int kMaxDeferred = 256;        // per-workgroup deferred pieces kept in LDS
constexpr int kMaxOwnChunks = 8;         // draw chunks per workgroup
constexpr int kPieceUnroll = 2;          // 16-byte vectors per thread per batch (two batches in flight)

struct FPiece {          // one row piece
    float m;             // piece max (sampled) / argmax value (greedy)
    int g;               // piece argmax (greedy)
    double z;            // sum of exp2((l - m) * c) over the piece
};

struct DrawParams {      // per request, written before its publication word
    double z32;
    float m;
    float v;
    int pos;
    int pad[3];
};

struct FusedParams {
    Params p;
    long vpr;                        // 16-byte vectors per row
    int pieces;                      // P: pieces per row (<= kMaxPieces)
    int items;                       // (gamma + 1) * batch * P
    int chunks;                      // C: draw chunks per request
    uint32_t epoch;                  // per-call tag of the publication words (never 0)
    FPiece* fpieces;                 // [rows][kMaxPieces]
    DrawParams* dparams;             // [batch]
    unsigned long long* words;       // [batch] (epoch << 32) | (kind << 30) | row
    unsigned long long* state;       // [batch] (accepted << 32) | decided; 0 between calls
};

// Per-request decision word: bit i of `decided` = row i's decision is made
// (bit gamma_b: the bonus row is done); bit i of `accepted` = draft i accepted.
struct ReqState {
    uint32_t decided, accepted;
};

__device__ __forceinline__ ReqState unpack_state(unsigned long long w) {
    ReqState s;
    s.decided = static_cast<uint32_t>(w);
    s.accepted = static_cast<uint32_t>(w >> 32);
    return s;
}
__device__ __forceinline__ unsigned long long pack_state(ReqState s) {
    return (static_cast<unsigned long long>(s.accepted) << 32) | s.decided;
}
// First rejection k (or gamma_b when all drafts are accepted and the bonus row
// is done); -1 while undecidable.
__device__ __forceinline__ int resolved_at(ReqState s, int gb) {
    const uint32_t ok = s.decided & s.accepted;
    const int k = (ok == 0xffffffffu) ? 32 : __builtin_ctz(~ok);   // first position not decided-and-accepted
    if (k < gb) return ((s.decided >> k) & 1u) ? k : -1;
    return ((s.decided >> gb) & 1u) ? gb : -1;
}

struct ItemMap {
    int i, b, p;         // position, request, piece
    int gb, d0;          // gamma_b, first draft row
    bool exists;
};

__device__ __forceinline__ ItemMap map_item(const FusedParams& F, int j) {
    const Params& P = F.p;
    ItemMap m;
    m.p = j % F.pieces;
    const int rem = j / F.pieces;
    m.b = rem % P.batch;
    m.i = rem / P.batch;
    if (P.offsets) {
        const int o0 = P.offsets[m.b], o1 = P.offsets[m.b + 1];
        m.d0 = o0;
        m.gb = o1 - o0;
        const bool ok = (o0 >= 0) && (o1 <= P.total_draft) && (m.gb >= 0) && (m.gb <= P.gamma);
        if (!ok && threadIdx.x == 0 && m.i == 0 && m.p == 0) flag_error(P.err, kErrOffsets);
        m.exists = ok && (m.i <= m.gb);
    } else {
        m.d0 = m.b * P.gamma;
        m.gb = P.gamma;
        m.exists = (m.i <= m.gb);
    }
    return m;
}

struct FusedShared {
    DrawShared d;
    int defer[kMaxDeferred];
    int ndefer;
    unsigned long long word;
    unsigned long long st;
    unsigned long long words[kMaxOwnChunks];
    int own[kMaxOwnChunks];          // this workgroup's pending draw chunks
    int nown;
    int flag;
    int k;
    int gk;
    float mk;
    double zk;
};

// Streams vectors [v0, v1) of an aligned row: two batches of kPieceUnroll
// vectors in flight per thread, full batches without per-vector checks.
template <typename E>
__device__ __forceinline__ void stream_piece(const v4u* vp, long v0, long v1, bool greedy, float c,
                                             float& m_out, int& g_out, double& z_out, RedScratch& red) {
    constexpr int U = kPieceUnroll;
    constexpr int EB = U * E::kPerVec;
    const int tid = threadIdx.x;
    const long span = v1 - v0 - tid;
    const int n = span > 0 ? static_cast<int>((span + kThreads - 1) / kThreads) : 0;
    const int nfull = n / U * U;
    const v4u* p0 = vp + v0 + tid;
    float mt = -INFINITY;
    double st = 0.0;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    auto consume = [&](const v4u* X, int j0, int cnt) {
        float f[EB];
#pragma unroll
        for (int u = 0; u < U; ++u) E::decode(X[u], f + u * E::kPerVec);
        if (!greedy) {
            accumulate_batch<EB>(f, c, mt, st);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u < cnt) {
                    const int x0 = static_cast<int>((v0 + tid + (long)(j0 + u) * kThreads) * E::kPerVec);
#pragma unroll
                    for (int k = 0; k < E::kPerVec; ++k) argmax_merge(bv, bi, f[u * E::kPerVec + k], x0 + k);
                }
            }
        }
    };
    v4u A[U], B[U];
    if (nfull > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) A[u] = __builtin_nontemporal_load(p0 + (long)u * kThreads);
    }
    int jb = 0;
    for (; jb + U < nfull; jb += 2 * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) B[u] = __builtin_nontemporal_load(p0 + (long)(jb + U + u) * kThreads);
        consume(A, jb, U);
        if (jb + 2 * U < nfull) {
#pragma unroll
            for (int u = 0; u < U; ++u) A[u] = __builtin_nontemporal_load(p0 + (long)(jb + 2 * U + u) * kThreads);
        }
        consume(B, jb + U, U);
    }
    if (jb < nfull) consume(A, jb, U);
    if (nfull < n) {
        // tail batch: vectors past this thread's range read as -inf
        v4u X[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            X[u] = (nfull + u < n) ? __builtin_nontemporal_load(p0 + (long)(nfull + u) * kThreads) : v4u(E::kNegInfWord);
        consume(X, nfull, n - nfull);
    }
    if (!greedy) {
        const float M = wg_max(mt, red);
        double zs = 0.0;
        if (mt > -INFINITY)
            zs = st * exp2((static_cast<double>(mt) - static_cast<double>(M)) * static_cast<double>(c));
        z_out = wg_sum(zs, red);
        m_out = M;
        g_out = -1;
    } else {
        wg_argmax(bv, bi, red);
        m_out = bv;
        g_out = bi;
        z_out = 0.0;
    }
}

// Resolve request b at position k (uniform call): outputs, then the draw
// publication.  mk, zk, gk are row k's statistics.
template <typename E>
__device__ __forceinline__ void fused_resolve(const FusedParams& F, int b, int gb, int d0, int k, float T, float mk, double zk,
                              int gk) {
    const Params& P = F.p;
    const int tid = threadIdx.x;
    const int Gm = P.gamma;
    const bool greedy = !(T > 0.0f);
    // Outputs go straight to the device-coherent level: another workgroup (on
    // another XCD) writes the drawn token into column k, and two L2s must never
    // hold dirty copies of the same bytes.  Column k of a sampled request is
    // left to that workgroup.
    if (tid <= Gm && (greedy || tid != k)) {
        int tok = -1;
        if (tid < k) tok = P.ids[d0 + tid];
        else if (tid == k) tok = gk;
        st_coherent(&P.out_tokens[(size_t)b * (Gm + 1) + tid], tok);
    }
    if (tid == 0) {
        st_coherent(&P.out_num[b], k);
        unsigned long long word = static_cast<unsigned long long>(F.epoch) << 32;
        if (!greedy) {
            const int kind = k < gb ? kDrawResidual : kDrawBonus;
            DrawParams* dp = &F.dparams[b];
            st_coherent(&dp->z32, zk);
            st_coherent(&dp->m, mk);
            st_coherent(&dp->v, P.uniforms[(size_t)b * (Gm + 2) + (k < gb ? Gm : Gm + 1)]);
            st_coherent(&dp->pos, k);
            word |= (static_cast<unsigned long long>(kind) << 30) | static_cast<unsigned long long>(d0 + b + k);
        }
        wait_stores();
        st_coherent(&F.words[b], word);
    }
}

// One row piece: stream, publish; the last piece merges the row, decides, and
// may resolve the request.  Uniform call; ends with the workgroup in step.
template <typename E>
__device__ __forceinline__ void fused_piece(const FusedParams& F, const ItemMap& it, FusedShared& sh) {
    const Params& P = F.p;
    const int tid = threadIdx.x;
    const int V = P.vocab;
    const int b = it.b, i = it.i, gb = it.gb, d0 = it.d0;
    const long t = (long)d0 + b + i;
    const float T = P.temperature[b];
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : static_cast<float>(kLog2e / static_cast<double>(T));
    const int NP = F.pieces;
    const long v0 = (long)it.p * F.vpr / NP, v1 = (long)(it.p + 1) * F.vpr / NP;
    int xdraft = -1;
    if (tid == 0 && i < gb && it.p == 0) xdraft = P.ids[d0 + i];

    const typename E::T* row = static_cast<const typename E::T*>(P.logits) + (size_t)t * V;
    float pm;
    int pg;
    double pz;
    stream_piece<E>(reinterpret_cast<const v4u*>(row), v0, v1, greedy, c, pm, pg, pz, sh.d.red);

    if (tid == 0) {
        FPiece* pp = &F.fpieces[(size_t)t * kMaxPieces + it.p];
        st_coherent(&pp->m, pm);
        st_coherent(&pp->g, pg);
        st_coherent(&pp->z, pz);
        if (it.p == 0) {
            // piece 0 also gathers the drafted token (and its logit and q) for the accept test
            float lx = 0.0f, qx = 0.0f;
            int xs = -1;
            if (i < gb) {
                if (xdraft >= 0 && xdraft < V) {
                    xs = xdraft;
                    if (!greedy) {
                        lx = E::load1(row, xdraft);
                        qx = P.q[(size_t)(d0 + i) * V + xdraft];
                    }
                } else {
                    flag_error(P.err, kErrDraftId);
                }
            }
            RowStat* rp = &P.rows[t];
            st_coherent(&rp->lx, lx);
            st_coherent(&rp->qx, qx);
            st_coherent(&rp->x, xs);
        }
        const int last = (arrive(&P.row_cnt[t]) == static_cast<uint32_t>(NP - 1));
        if (last) reset_counter(&P.row_cnt[t]);
        sh.flag = last;
    }
    __syncthreads();
    const int last = sh.flag;
    __syncthreads();
    if (!last) return;

    // ---- merge the row (lane s of wave 0 holds piece s) and decide
    if (tid < 64) {
        const int s = tid;
        float m = -INFINITY;
        int g = 0x7fffffff;
        double z = 0.0;
        if (s < NP) {
            const FPiece* pp = &F.fpieces[(size_t)t * kMaxPieces + s];
            m = ld_coherent(&pp->m);
            g = ld_coherent(&pp->g);
            z = ld_coherent(&pp->z);
        }
        float M = m;
        int Gi = g;
        wave_argmax(M, Gi);
        double zt = 0.0;
        if (!greedy && s < NP && m > -INFINITY)
            zt = z * exp2((static_cast<double>(m) - static_cast<double>(M)) * static_cast<double>(c));
        zt = wave_sum(zt);
        if (tid == 0) {
            const RowStat* rp = &P.rows[t];
            const float lx = ld_coherent(&rp->lx);
            const float qx = ld_coherent(&rp->qx);
            const int xv = ld_coherent(&rp->x);
            RowStat* wp = &P.rows[t];
            const double Z = greedy ? 0.0 : zt;
            st_coherent(&wp->m, M);
            st_coherent(&wp->g, Gi);
            st_coherent(&wp->z, Z);
            if (P.diag_m) st_coherent(&P.diag_m[t], M);
            if (P.diag_z) st_coherent(&P.diag_z[t], Z);
            // this row's decision bits
            const uint32_t dbit = 1u << i;
            uint32_t abit = 0u;
            if (i < gb) {
                bool acc;
                if (greedy) {
                    acc = (xv == Gi);
                    if (P.diag_r) st_coherent(&P.diag_r[d0 + i], __uint_as_float(0x7fc00000u));
                } else {
                    const double invT = 1.0 / static_cast<double>(T);
                    const double px = exp((static_cast<double>(lx) - static_cast<double>(M)) * invT) / zt;
                    const double r = px / fmax(static_cast<double>(qx), kQFloor);
                    const double u = static_cast<double>(P.uniforms[(size_t)b * (P.gamma + 2) + i]);
                    acc = (xv >= 0) && (u < fmin(1.0, r));
                    if (P.diag_r) st_coherent(&P.diag_r[d0 + i], static_cast<float>(r));
                }
                if (acc) abit = 1u << i;
            }
            wait_stores();       // row statistics are visible before the decision is
            unsigned long long* sp = &F.state[b];
            unsigned long long old = ld_coherent(sp);
            const uint32_t all = (gb >= 31) ? 0xffffffffu : ((2u << gb) - 1u);   // rows 0..gb
            ReqState os, ns;
            while (true) {
                os = unpack_state(old);
                ns.decided = os.decided | dbit;
                ns.accepted = os.accepted | abit;
                // the update that completes the request's rows leaves the word cleared
                const unsigned long long nw = (ns.decided == all) ? 0ull : pack_state(ns);
                if (__hip_atomic_compare_exchange_strong(sp, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT))
                    break;
            }
            const int k_old = resolved_at(os, gb), k_new = resolved_at(ns, gb);
            sh.k = (k_old < 0 && k_new >= 0) ? k_new : -1;
            sh.mk = M;
            sh.zk = Z;
            sh.gk = Gi;
        }
    }
    __syncthreads();
    const int k = sh.k;
    if (k >= 0) {
        // row k's statistics: this row's, or published before its decision
        float mk = sh.mk;
        double zk = sh.zk;
        int gk = sh.gk;
        if (k != i) {
            const RowStat* rk = &P.rows[(size_t)d0 + b + k];
            mk = ld_coherent(&rk->m);
            zk = ld_coherent(&rk->z);
            gk = ld_coherent(&rk->g);
        }
        fused_resolve<E>(F, b, gb, d0, k, T, mk, zk, gk);
    }
    __syncthreads();
}

// One draw chunk: blocks [c NB / C, (c+1) NB / C) of request b's draw row;
// the last chunk of the request runs the select.  Uniform call.
template <typename E>
__device__ __forceinline__ void fused_chunk(const FusedParams& F, int cid, unsigned long long word, FusedShared& sh) {
    const Params& P = F.p;
    const int tid = threadIdx.x;
    const int C = F.chunks;
    const int b = cid / C;
    const int c = cid - b * C;
    const int NB = P.nblocks;
    const int kind = static_cast<int>((word >> 30) & 3u);
    const int row = static_cast<int>(word & 0x3fffffffu);
    BlockRec* recs = P.recs + (size_t)b * NB;
    DrawRow<E> d;
    const bool work = (kind == kDrawResidual || kind == kDrawBonus) &&
                      row < P.total_draft + P.batch && row - b >= 0;
    if (work) {
        const DrawParams* dp = &F.dparams[b];
        init_draw_row<E>(d, P, kind, row, row - b, ld_coherent(&dp->pos), ld_coherent(&dp->v),
                         ld_coherent(&dp->m), ld_coherent(&dp->z32), P.temperature[b]);
        const int j0 = static_cast<int>((long)c * NB / C), j1 = static_cast<int>((long)(c + 1) * NB / C);
        draw_blocks<E>(d, P.vocab, recs, j0, kWaves, j1, sh.d.tab);
    }
    wait_stores();
    __syncthreads();
    if (tid == 0) {
        const int last = (arrive(&P.draw_cnt[b]) == static_cast<uint32_t>(C - 1));
        if (last) reset_counter(&P.draw_cnt[b]);
        sh.flag = last;
    }
    __syncthreads();
    const int last = sh.flag;
    __syncthreads();
    if (last && work) {
        const int y = draw_select<E>(d, P.vocab, NB, recs, sh.d, P.err);
        if (tid == 0 && d.pos >= 0 && d.pos <= P.gamma)
            st_coherent(&P.out_tokens[(size_t)b * (P.gamma + 1) + d.pos], y);
    }
    __syncthreads();
}

// Thread 0 re-reads the publication words of this workgroup's pending chunks;
// the workgroup then takes every published one (no waiting).  Uniform call.
template <typename E>
__device__ __forceinline__ void take_ready_chunks(const FusedParams& F, FusedShared& sh) {
    const int tid = threadIdx.x;
    if (sh.nown == 0) return;
    if (tid == 0)
        for (int q = 0; q < sh.nown; ++q) sh.words[q] = ld_coherent(&F.words[sh.own[q] / F.chunks]);
    __syncthreads();
    for (int q = 0; q < sh.nown; ++q) {
        const unsigned long long word = sh.words[q];
        if (static_cast<uint32_t>(word >> 32) != F.epoch) continue;
        const int cid = sh.own[q];
        __syncthreads();
        if (tid == 0) {                   // drop it from the pending list (keep the order of the rest)
            for (int r = q; r + 1 < sh.nown; ++r) { sh.own[r] = sh.own[r + 1]; sh.words[r] = sh.words[r + 1]; }
            --sh.nown;
        }
        __syncthreads();
        fused_chunk<E>(F, cid, word, sh);
        --q;
    }
    __syncthreads();
}

template <typename E>
__global__ __launch_bounds__(kThreads) void fused_step_kernel(FusedParams F) {
    __shared__ FusedShared sh;
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    const int G = gridDim.x;
    if (tid < 64) sh.d.tab[tid] = kExp2Table[tid];
    if (tid == 0) { sh.ndefer = 0; sh.flag = 0; }

    // this workgroup's draw chunks (the host keeps them to at most kMaxOwnChunks)
    if (tid == 0) {
        int n = 0;
        for (int cid = w; cid < F.p.batch * F.chunks && n < kMaxOwnChunks; cid += G) sh.own[n++] = cid;
        sh.nown = n;
    }
    __syncthreads();

    // ---- row pieces in position-major order; pieces of resolved requests set aside
    unsigned long long next_st = 0ull;        // thread 0: request word for the next item
    if (tid == 0 && w < F.items) {
        const ItemMap it = map_item(F, w);
        if (it.exists && it.i > 0) next_st = ld_coherent(&F.state[it.b]);
    }
    for (int j = w; j < F.items; j += G) {
        const ItemMap it = map_item(F, j);
        if (tid == 0) {
            sh.st = next_st;
            next_st = 0ull;
            if (j + G < F.items) {                // prefetch the next item's request word
                const ItemMap nx = map_item(F, j + G);
                if (nx.exists && nx.i > 0) next_st = ld_coherent(&F.state[nx.b]);
            }
        }
        __syncthreads();
        const ReqState s = unpack_state(sh.st);
        __syncthreads();
        if (!it.exists) continue;
        const int k = resolved_at(s, it.gb);
        bool now = true;
        if (k >= 0 && k < it.i) {
            if (tid == 0) {
                if (sh.ndefer < kMaxDeferred) { sh.defer[sh.ndefer++] = j; sh.flag = 1; }
                else sh.flag = 0;               // list full: stream it now
            }
            __syncthreads();
            now = (sh.flag == 0);
            __syncthreads();
        }
        if (now) fused_piece<E>(F, it, sh);
        take_ready_chunks<E>(F, sh);
    }
    // ---- deferred pieces (statistics only), interleaved with published chunks
    const int nd = sh.ndefer;
    for (int q = 0; q < nd; ++q) {
        const ItemMap it = map_item(F, sh.defer[q]);
        fused_piece<E>(F, it, sh);
        take_ready_chunks<E>(F, sh);
    }
    // ---- remaining chunks: wait (bounded) for their publication
    for (;;) {
        const int pending = sh.nown;     // every wave reads the count before thread 0 changes it
        __syncthreads();
        if (pending == 0) break;
        if (tid == 0) {
            const unsigned long long* wp = &F.words[sh.own[0] / F.chunks];
            unsigned long long word = ld_coherent(wp);
            int spins = 0;
            // a publication can only be missing when a row was rejected for
            // inconsistent offsets; stop waiting as soon as that is flagged
            while (static_cast<uint32_t>(word >> 32) != F.epoch && spins < kSpinLimit &&
                   (ld_coherent(F.p.err) & kErrOffsets) == 0u) {
                __builtin_amdgcn_s_sleep(2);
                word = ld_coherent(wp);
                ++spins;
            }
            if (static_cast<uint32_t>(word >> 32) != F.epoch) {
                flag_error(F.p.err, kErrOffsets);
                word = static_cast<unsigned long long>(F.epoch) << 32;   // treat as no draw
            }
            sh.word = word;
            sh.flag = sh.own[0];
            for (int r = 0; r + 1 < sh.nown; ++r) sh.own[r] = sh.own[r + 1];
            --sh.nown;
        }
        __syncthreads();
        const unsigned long long word = sh.word;
        const int cid = sh.flag;
        __syncthreads();
        fused_chunk<E>(F, cid, word, sh);
        take_ready_chunks<E>(F, sh);
    }
}

}  // namespace sv
