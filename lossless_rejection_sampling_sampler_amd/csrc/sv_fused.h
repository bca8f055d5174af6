// One-launch verify step for 16-byte aligned rows (the fast path).
//
// Method: the spec-decoding page at dpshk.com/news/5598276, sections 3.1-3.2,
// 5.2-5.3 and 8 (see sv_device.h); this file only changes how the same work is
// scheduled on the chip.
//
// A persistent, cooperatively launched grid (every workgroup resident at once)
// runs the whole step:
//
//   rows     The flattened [rows x 16-byte vectors] stream is cut into a few
//            rounds of consecutive rows; within a round every workgroup takes
//            one equal contiguous slice.  A slice yields one partial (max and
//            fp32-exponential sum, or argmax) per row piece.  The last piece of
//            a row bumps the request's row counter; the last row of a request
//            merges all pieces of the request's rows, runs the accept tests,
//            writes the outputs and publishes the draw (parameters first, then
//            one 64-bit word carrying the call's epoch and the draw row).
//   draws    Every request's draw row is cut into C chunks of 512-token blocks;
//            chunk i of the call belongs to workgroup i mod grid.  Between
//            slices a workgroup takes whichever of its chunks are published
//            (it never waits while it still has slices to stream), so draws of
//            requests resolved in early rounds overlap the streaming of later
//            rounds.  After its last slice a workgroup waits (bounded) for its
//            remaining chunks.  The last chunk of a request to finish runs the
//            select (exact fp64 normaliser, block scan, token scan).
//
// Requests resolve round by round because rounds follow the row order, and the
// only waits are for publications made by workgroups that never wait
// themselves, so the grid always drains.
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kSpinLimit = 1 << 20;      // bounded wait for a publication (about a second)

struct FPiece {          // one row piece of the fused step
    float m;             // piece max (sampled) / argmax value (greedy)
    int g;               // piece argmax (greedy)
    double z;            // sum of exp2((l - m) * c) over the piece
    float lx;            // piece 0 only: logit of the drafted token
    float qx;            // piece 0 only: q of the drafted token
    int x;               // piece 0 only: drafted token (-1 if invalid / none)
    int pad;
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
    long nv, vpr;                    // flattened stream: total vectors, vectors per row
    int nrounds;                     // round k covers vectors [nv k / nrounds, nv (k+1) / nrounds)
    int chunks;                      // draw chunks per request
    uint32_t epoch;                  // per-call tag of the publication words
    FPiece* pieces;                  // [rows][kMaxPieces]
    DrawParams* dparams;             // [batch]
    unsigned long long* words;       // [batch] (epoch << 32) | (kind << 30) | row
};

__device__ __forceinline__ long round_bound(const FusedParams& F, int k) {
    return F.nv * k / F.nrounds;
}

// Slice id (round * grid + workgroup) owning flattened vector v.
__device__ __forceinline__ int slice_of(const FusedParams& F, long v, int G) {
    const int k = range_owner(v, F.nv, F.nrounds);
    const long b0 = round_bound(F, k);
    return k * G + range_owner(v - b0, round_bound(F, k + 1) - b0, G);
}

__device__ __forceinline__ int row_pieces(const FusedParams& F, long t, int G) {
    return slice_of(F, (t + 1) * F.vpr - 1, G) - slice_of(F, t * F.vpr, G) + 1;
}

struct FusedShared {
    DrawShared d;
    unsigned long long word;
    int flag;
    int k;
    float dm;
    double dz;
};

// Streams vectors [v0, v1) of an aligned row; returns the workgroup-reduced
// (max, fp32-exponential sum) or, for greedy rows, (max, argmax).
template <typename E>
__device__ __forceinline__ void stream_piece(const v4u* vp, long v0, long v1, bool greedy, float c,
                                             float& m_out, int& g_out, double& z_out, RedScratch& red) {
    const int tid = threadIdx.x;
    const long span = v1 - v0 - tid;
    const int n = span > 0 ? static_cast<int>((span + kThreads - 1) / kThreads) : 0;
    const long first = v0 + tid;
    constexpr int EB = kRowUnroll * E::kPerVec;
    v4u A[kRowUnroll];
    if (n > 0) load_batch<E>(A, vp, first, n);
    if (!greedy) {
        float mt = -INFINITY;
        double st = 0.0;
        for (int jb = 0; jb < n; jb += kRowUnroll) {
            // the next batch is in flight while this one is reduced
            v4u Nx[kRowUnroll];
            if (jb + kRowUnroll < n)
                load_batch<E>(Nx, vp, first + (long)(jb + kRowUnroll) * kThreads, n - jb - kRowUnroll);
            float f[EB];
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) E::decode(A[u], f + u * E::kPerVec);
            accumulate_batch<EB>(f, c, mt, st);
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) A[u] = Nx[u];
        }
        const float M = wg_max(mt, red);
        double zs = 0.0;
        if (mt > -INFINITY)
            zs = st * exp2((static_cast<double>(mt) - static_cast<double>(M)) * static_cast<double>(c));
        z_out = wg_sum(zs, red);
        m_out = M;
        g_out = -1;
    } else {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int jb = 0; jb < n; jb += kRowUnroll) {
            v4u Nx[kRowUnroll];
            if (jb + kRowUnroll < n)
                load_batch<E>(Nx, vp, first + (long)(jb + kRowUnroll) * kThreads, n - jb - kRowUnroll);
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                float f[E::kPerVec];
                E::decode(A[u], f);
                const int x0 = static_cast<int>((first + (long)(jb + u) * kThreads) * E::kPerVec);
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) argmax_merge(bv, bi, f[k], x0 + k);
            }
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) A[u] = Nx[u];
        }
        wg_argmax(bv, bi, red);
        m_out = bv;
        g_out = bi;
        z_out = 0.0;
    }
}

// Resolve request b once all its rows' pieces are in.  Each row is merged by a
// group of 16 lanes (one lane per piece, shuffle reductions inside the group);
// the group leader runs the row's accept test.
template <typename E>
__device__ void fused_resolve(const FusedParams& F, const RowMap& rm, float T, FusedShared& sh, int G) {
    static_assert(kMaxPieces == 16, "one 16-lane group per row");
    const Params& P = F.p;
    const int tid = threadIdx.x;
    const int b = rm.b, gb = rm.gb;
    const int Gm = P.gamma;
    const int t0 = rm.d0 + b;
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : static_cast<float>(kLog2e / static_cast<double>(T));
    const int s = tid & 15;                        // piece handled by this lane
    if (tid == 0) sh.k = gb;
    __syncthreads();
    for (int j0 = 0; j0 <= gb; j0 += kThreads / 16) {
        const int j = j0 + (tid >> 4);             // row of this lane's group
        const bool active = (j <= gb);
        float pm = -INFINITY;
        int pg = 0x7fffffff;
        double pz = 0.0;
        float lx = 0.0f, qx = 0.0f;
        int xv = -1;
        const long t = t0 + j;
        if (active) {
            const int np = row_pieces(F, t, G);
            const FPiece* pp = &F.pieces[(size_t)t * kMaxPieces + s];
            if (s < np) {
                pm = ld_coherent(&pp->m);
                pg = ld_coherent(&pp->g);
                pz = ld_coherent(&pp->z);
            }
            if (s == 0) {
                lx = ld_coherent(&pp->lx);
                qx = ld_coherent(&pp->qx);
                xv = ld_coherent(&pp->x);
            }
        }
        // group (16-lane) reductions
        float m = pm;
        int g = pg;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
            const float m2 = __shfl_xor(m, o, 64);
            const int g2 = __shfl_xor(g, o, 64);
            argmax_merge(m, g, m2, g2);
        }
        double zt = 0.0;
        if (!greedy && pm > -INFINITY)
            zt = pz * exp2((static_cast<double>(pm) - static_cast<double>(m)) * static_cast<double>(c));
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) zt += __shfl_xor(zt, o, 64);
        if (active && s == 0) {
            if (P.diag_m) st_coherent(&P.diag_m[t], m);
            if (P.diag_z) st_coherent(&P.diag_z[t], greedy ? 0.0 : zt);
            sh.d.w[j] = zt;                        // row Z for the draw
            sh.d.list[j] = g;                      // row argmax for greedy outputs
            reinterpret_cast<float*>(sh.d.w + kMaxDrawBlocks / 2)[j] = m;
            if (j < gb) {
                bool acc;
                if (greedy) {
                    acc = (P.ids[rm.d0 + j] == g);
                    if (P.diag_r) st_coherent(&P.diag_r[rm.d0 + j], __uint_as_float(0x7fc00000u));
                } else {
                    const double invT = 1.0 / static_cast<double>(T);
                    const double px = exp((static_cast<double>(lx) - static_cast<double>(m)) * invT) / zt;
                    const double r = px / fmax(static_cast<double>(qx), kQFloor);
                    const double u = static_cast<double>(P.uniforms[(size_t)b * (Gm + 2) + j]);
                    acc = (xv >= 0) && (u < fmin(1.0, r));
                    if (P.diag_r) st_coherent(&P.diag_r[rm.d0 + j], static_cast<float>(r));
                }
                if (!acc) atomicMin(&sh.k, j);
            }
        }
    }
    __syncthreads();
    const int k = sh.k;
    // Outputs go straight to the device-coherent level: another workgroup (on
    // another XCD) writes the drawn token into column k of the same row, and two
    // L2s must never hold dirty copies of it.  Column k of a sampled request is
    // left to that workgroup.
    if (tid <= Gm && (greedy || tid != k)) {
        int tok = -1;
        if (tid < k) tok = P.ids[rm.d0 + tid];
        else if (tid == k) tok = sh.d.list[k];
        st_coherent(&P.out_tokens[(size_t)b * (Gm + 1) + tid], tok);
    }
    if (tid == 0) {
        st_coherent(&P.out_num[b], k);
        unsigned long long word = (static_cast<unsigned long long>(F.epoch) << 32);
        if (!greedy) {
            const int kind = k < gb ? kDrawResidual : kDrawBonus;
            DrawParams* dp = &F.dparams[b];
            st_coherent(&dp->z32, sh.d.w[k]);
            st_coherent(&dp->m, reinterpret_cast<const float*>(sh.d.w + kMaxDrawBlocks / 2)[k]);
            st_coherent(&dp->v, P.uniforms[(size_t)b * (Gm + 2) + (k < gb ? Gm : Gm + 1)]);
            st_coherent(&dp->pos, k);
            word |= (static_cast<unsigned long long>(kind) << 30) | static_cast<unsigned long long>(t0 + k);
        }
        wait_stores();
        st_coherent(&F.words[b], word);
    }
    __syncthreads();
}

// Streams one slice piece of row t and hands the row / request on when complete.
template <typename E>
__device__ void fused_piece(const FusedParams& F, long t, long v0, long v1, int piece, int npieces,
                            FusedShared& sh, int G) {
    const Params& P = F.p;
    const int tid = threadIdx.x;
    const int V = P.vocab;
    const RowMap rm = map_row(P, static_cast<int>(t), sh.d.red);
    if (!rm.ok) {
        if (tid == 0 && piece == 0) flag_error(P.err, kErrOffsets);
        return;
    }
    if (piece >= kMaxPieces || npieces > kMaxPieces) {     // excluded by the launch geometry
        if (tid == 0) flag_error(P.err, kErrOffsets);
        return;
    }
    const int b = rm.b, i = rm.i, gb = rm.gb;
    const float T = P.temperature[b];
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : static_cast<float>(kLog2e / static_cast<double>(T));
    const bool gather = (piece == 0) && !greedy && (i < gb);
    int xdraft = -1;
    if (tid == 0 && gather) xdraft = P.ids[rm.d0 + i];

    const typename E::T* row = static_cast<const typename E::T*>(P.logits) + (size_t)t * V;
    const v4u* vp = reinterpret_cast<const v4u*>(row);
    float pm;
    int pg;
    double pz;
    stream_piece<E>(vp, v0, v1, greedy, c, pm, pg, pz, sh.d.red);

    if (tid == 0) {
        FPiece* pp = &F.pieces[(size_t)t * kMaxPieces + piece];
        st_coherent(&pp->m, pm);
        st_coherent(&pp->g, pg);
        st_coherent(&pp->z, pz);
        if (piece == 0) {
            float lx = 0.0f, qx = 0.0f;
            int xs = -1;
            if (gather) {
                if (xdraft >= 0 && xdraft < V) {
                    xs = xdraft;
                    lx = E::load1(row, xdraft);
                    qx = P.q[(size_t)(rm.d0 + i) * V + xdraft];
                } else {
                    flag_error(P.err, kErrDraftId);
                }
            }
            st_coherent(&pp->lx, lx);
            st_coherent(&pp->qx, qx);
            st_coherent(&pp->x, xs);
        }
        int last = 0;
        if (arrive(&P.row_cnt[t]) == static_cast<uint32_t>(npieces - 1)) {
            reset_counter(&P.row_cnt[t]);
            if (arrive(&P.req_cnt[b]) == static_cast<uint32_t>(gb)) {
                reset_counter(&P.req_cnt[b]);
                last = 1;
            }
        }
        sh.flag = last;
    }
    __syncthreads();
    const int last = sh.flag;
    __syncthreads();
    if (last) fused_resolve<E>(F, rm, T, sh, G);
}

// One draw chunk: blocks [c NB / C, (c+1) NB / C) of request b's draw row;
// the last chunk of the request runs the select.
template <typename E>
__device__ void fused_chunk(const FusedParams& F, int cid, unsigned long long word, FusedShared& sh) {
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
}

template <typename E>
__global__ __launch_bounds__(kThreads) void fused_step_kernel(FusedParams F) {
    __shared__ FusedShared sh;
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    const int G = gridDim.x;
    const int nch = F.p.batch * F.chunks;
    if (tid < 64) sh.d.tab[tid] = kExp2Table[tid];
    __syncthreads();

    int cursor = w;                    // this workgroup's next draw chunk: w, w + G, ...
    unsigned long long pending = 0;    // thread 0: prefetched publication word of `cursor`
    for (int k = 0; k < F.nrounds; ++k) {
        if (tid == 0 && cursor < nch) pending = ld_coherent(&F.words[cursor / F.chunks]);
        const long b0 = round_bound(F, k);
        const long L = round_bound(F, k + 1) - b0;
        const long a = b0 + (long)w * L / G, e = b0 + (long)(w + 1) * L / G;
        long r = a / F.vpr;
        for (long s0 = a; s0 < e; ++r) {
            const long rs = r * F.vpr, re = rs + F.vpr;
            const long s1 = e < re ? e : re;
            const int sf = slice_of(F, rs, G), sl = slice_of(F, re - 1, G);
            fused_piece<E>(F, r, s0 - rs, s1 - rs, k * G + w - sf, sl - sf + 1, sh, G);
            __syncthreads();
            s0 = s1;
        }
        // published chunks of this workgroup, without waiting
        while (true) {
            if (tid == 0) sh.word = (cursor < nch) ? pending : 0ull;
            __syncthreads();
            const unsigned long long word = sh.word;
            __syncthreads();
            if (cursor >= nch || static_cast<uint32_t>(word >> 32) != F.epoch) break;
            if (tid == 0 && cursor + G < nch) pending = ld_coherent(&F.words[(cursor + G) / F.chunks]);
            fused_chunk<E>(F, cursor, word, sh);
            cursor += G;
        }
    }
    // remaining chunks: wait (bounded) for their publication
    while (cursor < nch) {
        if (tid == 0) {
            const unsigned long long* wp = &F.words[cursor / F.chunks];
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
                flag_error(F.p.err, kErrOffsets);   // never published: inconsistent offsets
                word = static_cast<unsigned long long>(F.epoch) << 32;   // treat as no draw
            }
            sh.word = word;
        }
        __syncthreads();
        const unsigned long long word = sh.word;
        __syncthreads();
        fused_chunk<E>(F, cursor, word, sh);
        cursor += G;
    }
}

}  // namespace sv
