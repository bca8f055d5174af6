// One-launch verify step (the fast path for 16-byte aligned rows, gamma <= 30).
//
// Method: the spec-decoding page at dpshk.com/news/5598276, sections 3.1-3.2,
// 5.2-5.3 and 8 (see sv_device.h).  This file changes only how the same work
// is ordered on the chip, using the page's own observation (section 3.1, step
// 3) that verification stops at the first rejection: the draw of a request
// depends only on its rows up to that position.
//
// A persistent, cooperatively launched grid of single-wave workgroups (all
// resident at once; no workgroup barriers, latency is hidden by the other
// waves of the CU and by a software pipeline inside each wave), split into row
// waves and draw waves, runs:
//
//   row pieces  Every target row is cut into P <= 64 equal pieces.  Pieces are
//               taken in position-major order (position 0 of every request,
//               then position 1, ...), wave w taking items w, w + grid, ...
//               Each wave issues the loads of its next piece before it works
//               on the current one.  A piece yields (max, fp32-exponential sum)
//               or (max, argmax), stored as a record whose 8-byte halves all
//               carry the call's epoch, so a reader can tell a complete record
//               from a stale or half-written one without any store ordering.
//               The wave then counts the piece on the row's arrival counter and
//               reads the result one piece later: the wave that landed the
//               row's last piece merges it (one piece per lane, re-reading
//               records whose tags are not yet current) and makes the row's
//               accept decision; decisions are OR-ed into a per-request word by
//               CAS.  The update that makes the request decidable (first
//               rejection known, or every draft accepted and the bonus row done)
//               resolves it: outputs, then the draw parameters, then one 64-bit
//               publication word tagged with the epoch.  The update that
//               completes the request's rows clears the word for the next call.
//   deferral    A piece of a request already resolved at an earlier position is
//               not needed for the outputs (only for per-row statistics); the
//               wave sets it aside and streams it after its other pieces, so the
//               end of the step is non-critical streaming that covers the last
//               draws.
//   draws       Request b's draw row is cut into 2048-token blocks; block
//               (b, j) belongs to wave (b * NB + j) mod grid (lane q of a wave
//               holds its q-th block).  Between pieces a wave polls the
//               publication words of its pending blocks (the load is issued
//               before the piece and read after it) and works on the published
//               ones; at the end it waits (bounded) for the rest.  The wave that
//               lands a request's last block runs the select.
//
// The only waits are for publications and for records already sent, which
// are made by waves that never wait for anything but their own loads, so the
// grid always drains.
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kStepLanes = 64;           // one wave per workgroup
constexpr int kSpinLimit = 1 << 20;      // bounded wait for a publication (about a second)
constexpr int kTagSpin = 1 << 16;        // bounded re-reads of piece records already sent
constexpr int kMaxGammaStep = 30;        // decided bits 0..30 of the per-request word
constexpr int kMaxStepPieces = 64;       // pieces per row: one merge lane each
constexpr int kStepBatch = 2;            // 16-byte vectors per lane per load batch
constexpr int kPieceBatches = 6;         // batches per row piece: 12 vectors per lane
constexpr int kRing = 3;                 // batches in flight per row wave
constexpr int kPieceLaneVecs = kPieceBatches * kStepBatch;
constexpr int kPieceVecs = 64 * kPieceLaneVecs;   // 768 vectors (12 KiB) per piece
constexpr int kMaxDeferred = 128;        // deferred pieces per wave (LDS)
constexpr int kMaxOwnBlocks = 64;        // draw blocks per wave: one per lane

// One piece record: four 8-byte halves, each (value bits) | (epoch << 32).
//   h[0]  piece max (sampled) / argmax value (greedy), fp32 bits
//   h[1]  piece sum of exp2((l - m) * c) as fp32 (sampled) / argmax index (greedy)
//   h[2]  piece 0 of a draft row: logit of the drafted token, fp32 bits
//   h[3]  piece 0 of a draft row: q of the drafted token, fp32 bits
struct PieceRec {
    unsigned long long h[4];
};

struct DrawParams {      // per request, written before its publication word
    double z32;
    float m;
    float v;
    int pos;
    int pad[3];
};

struct StepParams {
    Params p;
    long vpr;                        // 16-byte vectors per row
    int pieces;                      // P: pieces per row (<= kMaxStepPieces)
    int items;                       // (gamma + 1) * batch * P
    uint32_t epoch;                  // per-call tag (never 0)
    int row_waves;                   // workgroups [0, row_waves) stream rows, the rest draw
    PieceRec* precs;                 // [rows][kMaxStepPieces]
    DrawParams* dparams;             // [batch]
    unsigned long long* words;       // [batch] (epoch << 32) | (kind << 30) | row
    unsigned long long* state;       // [batch] (accepted << 32) | decided; 0 between calls
};

__device__ __forceinline__ unsigned long long rdlane_u64(unsigned long long v, int l) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ unsigned long long tagged(uint32_t bits, uint32_t epoch) {
    return (static_cast<unsigned long long>(epoch) << 32) | bits;
}

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

// A candidate item with its request's word (and offsets, when given) loaded
// ahead of the decision whether to stream or defer it.
struct Cand {
    int j;                       // item index; >= items: none
    unsigned long long st;       // request word
    int o0, o1;                  // offsets[b], offsets[b + 1] (when given)
};

__device__ __forceinline__ Cand cand_load(const StepParams& S, int j) {
    const Params& P = S.p;
    Cand c;
    c.j = j;
    c.st = 0ull;
    c.o0 = c.o1 = 0;
    if (j < S.items) {
        const int b = (j / S.pieces) % P.batch;
        c.st = ld_coherent(&S.state[b]);
        if (P.offsets) {
            c.o0 = P.offsets[b];
            c.o1 = P.offsets[b + 1];
        }
    }
    return c;
}

// An item picked for streaming: its coordinates, its piece's vectors and the
// request's temperature (loaded one piece ahead).
struct Item {
    int j;                       // item index; -1: none
    int i, b, p, gb, d0;         // position, request, piece, gamma_b, first draft row
    float T;                     // temperature of the request
    int xd;                      // lane 0, piece 0 of a draft row: the drafted token
    const v4u* base;             // the piece's first vector
    int cnt;                     // vectors in the piece (<= kPieceVecs)
};

// Fills the item's coordinates from a candidate; false when the row does not
// exist (ragged gamma_b, or inconsistent offsets, which are flagged once).
__device__ __forceinline__ bool item_coords(const StepParams& S, int j, int o0, int o1, Item& it) {
    const Params& P = S.p;
    it.j = j;
    it.p = j % S.pieces;
    const int rem = j / S.pieces;
    it.b = rem % P.batch;
    it.i = rem / P.batch;
    if (P.offsets) {
        it.d0 = o0;
        it.gb = o1 - o0;
        const bool ok = (o0 >= 0) && (o1 <= P.total_draft) && (it.gb >= 0) && (it.gb <= P.gamma);
        if (!ok && threadIdx.x == 0 && it.i == 0 && it.p == 0) flag_error(P.err, kErrOffsets);
        return ok && it.i <= it.gb;
    }
    it.d0 = it.b * P.gamma;
    it.gb = P.gamma;
    return it.i <= it.gb;
}

// Issues the item's small loads (temperature, drafted token) and sets its piece.
template <typename E>
__device__ __forceinline__ void item_issue(const StepParams& S, Item& it) {
    const Params& P = S.p;
    const int lane = threadIdx.x & 63;
    it.T = P.temperature[it.b];
    it.xd = -1;
    if (lane == 0 && it.p == 0 && it.i < it.gb) it.xd = P.ids[it.d0 + it.i];
    const long t = (long)it.d0 + it.b + it.i;
    const long v0 = (long)it.p * kPieceVecs;
    it.base = reinterpret_cast<const v4u*>(static_cast<const typename E::T*>(P.logits) + (size_t)t * P.vocab) + v0;
    it.cnt = static_cast<int>(min((long)kPieceVecs, S.vpr - v0));
}

// Loads batch e of the item's piece into X: lane L takes vectors L + 64 n.
// Every load is issued (no branches, so the compiler can count them); vectors
// past the piece re-read its last one and are masked when consumed.
__device__ __forceinline__ void issue_batch(const Item& it, int e, v4u* X) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < kStepBatch; ++u) {
        const int v = min((e * kStepBatch + u) * 64 + lane, it.cnt - 1);
        X[u] = __builtin_nontemporal_load(it.base + v);
    }
}

// Per-lane running state of one piece.
struct PieceAcc {
    float mt;            // sampled: running max;  greedy: best value
    int bi;              // greedy: best index
    double st;           // sampled: running sum of exp2((l - mt) * c)
};

// Consumes batch e of the item's piece from X.
template <typename E>
__device__ __forceinline__ void consume_batch(const Item& it, int e, v4u* X, bool greedy, float c, const double* tab,
                                              PieceAcc& acc) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < kStepBatch; ++u)
        X[u] = ((e * kStepBatch + u) * 64 + lane < it.cnt) ? X[u] : v4u(E::kNegInfWord);
    if (!greedy) {
        // max pass, then the exponential pass decodes again (cheaper than
        // keeping the decoded batch in registers)
        float bm = -INFINITY;
#pragma unroll
        for (int u = 0; u < kStepBatch; ++u) {
            float f[E::kPerVec];
            E::decode(X[u], f);
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) bm = fmaxf(bm, f[k]);
        }
        if (bm > acc.mt) {
            if (acc.mt > -INFINITY)
                acc.st *= exp2_nonpos((static_cast<double>(acc.mt) - static_cast<double>(bm)) * static_cast<double>(c), tab);
            acc.mt = bm;
        }
        if (acc.mt > -INFINITY) {
            float sum = 0.0f;
#pragma unroll
            for (int u = 0; u < kStepBatch; ++u) {
                v4u x = X[u];
                asm volatile("" : "+v"(x));       // decode afresh, do not keep the first pass
                float f[E::kPerVec];
                E::decode(x, f);
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) sum += __builtin_amdgcn_exp2f((f[k] - acc.mt) * c);
                __builtin_amdgcn_sched_barrier(0);
            }
            acc.st += static_cast<double>(sum);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kStepBatch; ++u) {
            float f[E::kPerVec];
            E::decode(X[u], f);
            const int x0 = (it.p * kPieceVecs + (e * kStepBatch + u) * 64 + lane) * E::kPerVec;
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) argmax_merge(acc.mt, acc.bi, f[k], x0 + k);
        }
    }
}

// Resolve request b at position k (wave-uniform call): outputs, then the draw
// publication.  mk, zk, gk are row k's statistics.
__device__ __forceinline__ void step_resolve(const StepParams& S, int b, int gb, int d0, int k, float T, float mk,
                                             double zk, int gk) {
    const Params& P = S.p;
    const int lane = threadIdx.x & 63;
    const int Gm = P.gamma;
    const bool greedy = !(T > 0.0f);
    // Outputs go straight to the device-coherent level: another wave (on another
    // XCD) writes the drawn token into column k, and two L2s must never hold
    // dirty copies of the same bytes.  Column k of a sampled request is left to
    // that wave.
    if (lane <= Gm && (greedy || lane != k)) {
        int tok = -1;
        if (lane < k) tok = P.ids[d0 + lane];
        else if (lane == k) tok = gk;
        st_coherent(&P.out_tokens[(size_t)b * (Gm + 1) + lane], tok);
    }
    if (lane == 0) {
        st_coherent(&P.out_num[b], k);
        unsigned long long word = static_cast<unsigned long long>(S.epoch) << 32;
        if (!greedy) {
            const int kind = k < gb ? kDrawResidual : kDrawBonus;
            DrawParams* dp = &S.dparams[b];
            st_coherent(&dp->z32, zk);
            st_coherent(&dp->m, mk);
            st_coherent(&dp->v, P.uniforms[(size_t)b * (Gm + 2) + (k < gb ? Gm : Gm + 1)]);
            st_coherent(&dp->pos, k);
            word |= (static_cast<unsigned long long>(kind) << 30) | static_cast<unsigned long long>(d0 + b + k);
        }
        wait_stores();
        st_coherent(&S.words[b], word);
    }
}

// A piece whose arrival result is still in flight.
struct Arrival {
    bool valid;
    int i, b, gb, d0;
    float T;
    uint32_t old;                // lane 0: the counter before this arrival
};

// Finishes an arrival: the wave that landed the row's last piece merges the
// row, decides, and may resolve the request.  Wave-uniform call.
template <typename E>
__device__ __forceinline__ void finish_arrival(const StepParams& S, const Arrival& a, const double* tab) {
    const Params& P = S.p;
    const int lane = threadIdx.x & 63;
    const int NP = S.pieces;
    const long t = (long)a.d0 + a.b + a.i;
    if (rdlane(static_cast<int>(a.old), 0) != NP - 1) return;
    if (lane == 0) reset_counter(&P.row_cnt[t]);
    const int i = a.i, b = a.b, gb = a.gb, d0 = a.d0;
    const float T = a.T;
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : static_cast<float>(kLog2e / static_cast<double>(T));
    const int V = P.vocab;

    // ---- the row's records, lane s holding piece s (lane 0 also piece 0's gather)
    const PieceRec* rec = &S.precs[(size_t)t * kMaxStepPieces];
    const bool gather = (i < gb) && !greedy;
    int x = -1;
    if (lane == 0 && i < gb) x = P.ids[d0 + i];
    unsigned long long h0 = 0ull, h1 = 0ull, h2 = 0ull, h3 = 0ull;
    bool ok = true;
    for (int spin = 0;; ++spin) {
        if (lane < NP) {
            h0 = ld_coherent(&rec[lane].h[0]);
            h1 = ld_coherent(&rec[lane].h[1]);
        }
        if (lane == 0 && gather) {
            h2 = ld_coherent(&rec[0].h[2]);
            h3 = ld_coherent(&rec[0].h[3]);
        }
        bool stale = lane < NP && (static_cast<uint32_t>(h0 >> 32) != S.epoch ||
                                   static_cast<uint32_t>(h1 >> 32) != S.epoch);
        if (lane == 0 && gather)
            stale = stale || static_cast<uint32_t>(h2 >> 32) != S.epoch || static_cast<uint32_t>(h3 >> 32) != S.epoch;
        if (__ballot(stale) == 0ull) break;
        if (spin >= kTagSpin) {                  // never expected: the records were sent before the arrival
            ok = false;
            if (lane == 0) flag_error(P.err, kErrStalled);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    float m = -INFINITY;
    int g = 0x7fffffff;
    double z = 0.0;
    if (lane < NP && ok) {
        m = __uint_as_float(static_cast<uint32_t>(h0));
        if (greedy) g = static_cast<int>(static_cast<uint32_t>(h1));
        else z = static_cast<double>(__uint_as_float(static_cast<uint32_t>(h1)));
    }
    float M = m;
    int Gi = g;
    wave_argmax(M, Gi);
    double zt = 0.0;
    if (!greedy && lane < NP && m > -INFINITY)
        zt = z * exp2_nonpos((static_cast<double>(m) - static_cast<double>(M)) * static_cast<double>(c), tab);
    zt = wave_sum(zt);
    const double Z = greedy ? 0.0 : zt;
    int k = -1;
    if (lane == 0) {
        RowStat* rp = &P.rows[t];
        st_coherent(&rp->m, M);
        st_coherent(&rp->g, greedy ? Gi : -1);
        st_coherent(&rp->z, Z);
        if (P.diag_m) st_coherent(&P.diag_m[t], M);
        if (P.diag_z) st_coherent(&P.diag_z[t], Z);
        // this row's decision bits
        const uint32_t dbit = 1u << i;
        uint32_t abit = 0u;
        if (i < gb) {
            const bool xok = x >= 0 && x < V;
            if (!xok) flag_error(P.err, kErrDraftId);
            bool acc;
            if (greedy) {
                acc = xok && (x == Gi);
                if (P.diag_r) st_coherent(&P.diag_r[d0 + i], __uint_as_float(0x7fc00000u));
            } else {
                const double lx = static_cast<double>(__uint_as_float(static_cast<uint32_t>(h2)));
                const double qx = static_cast<double>(__uint_as_float(static_cast<uint32_t>(h3)));
                const double invT = 1.0 / static_cast<double>(T);
                const double px = exp((lx - static_cast<double>(M)) * invT) / zt;
                const double r = px / fmax(qx, kQFloor);
                const double u = static_cast<double>(P.uniforms[(size_t)b * (P.gamma + 2) + i]);
                acc = xok && (u < fmin(1.0, r));
                if (P.diag_r) st_coherent(&P.diag_r[d0 + i], static_cast<float>(r));
            }
            if (acc) abit = 1u << i;
        }
        wait_stores();           // row statistics are visible before the decision is
        unsigned long long* sp = &S.state[b];
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
        k = (k_old < 0 && k_new >= 0) ? k_new : -1;
    }
    k = rdlane(k, 0);
    if (k < 0) return;
    // row k's statistics: this row's, or published before its decision
    float mk = M;
    double zk = Z;
    int gk = Gi;
    if (k != i) {
        const RowStat* rk = &P.rows[(size_t)d0 + b + k];
        mk = ld_coherent(&rk->m);
        zk = ld_coherent(&rk->z);
        gk = ld_coherent(&rk->g);
    }
    step_resolve(S, b, gb, d0, k, T, mk, zk, gk);
}

// Ends a streamed piece: wave reductions, the tagged record (with the drafted
// token's logit and q for piece 0 of a draft row, gathered while the piece
// streamed) and the arrival on the row's counter, whose result is read one
// piece later.
template <typename E>
__device__ __forceinline__ Arrival item_finish(const StepParams& S, const Item& it, bool greedy, float c,
                                               const PieceAcc& acc, float lx, float qx, const double* tab) {
    const Params& P = S.p;
    const int lane = threadIdx.x & 63;
    const long t = (long)it.d0 + it.b + it.i;
    float pm;
    int pg;
    double pz = 0.0;
    if (!greedy) {
        pm = wave_max(acc.mt);
        double zs = 0.0;
        if (acc.mt > -INFINITY)
            zs = acc.st * exp2_nonpos((static_cast<double>(acc.mt) - static_cast<double>(pm)) * static_cast<double>(c), tab);
        pz = wave_sum(zs);
        pg = -1;
    } else {
        pm = acc.mt;
        pg = acc.bi;
        wave_argmax(pm, pg);
    }
    Arrival a;
    a.valid = true;
    a.i = it.i;
    a.b = it.b;
    a.gb = it.gb;
    a.d0 = it.d0;
    a.T = it.T;
    a.old = 0u;
    if (lane == 0) {
        PieceRec* pr = &S.precs[(size_t)t * kMaxStepPieces + it.p];
        const uint32_t v1 = greedy ? static_cast<uint32_t>(pg) : __float_as_uint(static_cast<float>(pz));
        st_coherent(&pr->h[0], tagged(__float_as_uint(pm), S.epoch));
        st_coherent(&pr->h[1], tagged(v1, S.epoch));
        if (it.p == 0 && it.i < it.gb && !greedy) {
            st_coherent(&pr->h[2], tagged(__float_as_uint(lx), S.epoch));
            st_coherent(&pr->h[3], tagged(__float_as_uint(qx), S.epoch));
        }
        // no wait for the stores: the merging wave checks the records' tags
        a.old = __hip_atomic_fetch_add(&P.row_cnt[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return a;
}

// One draw block (request b, block j); the wave that lands the request's last
// block runs the select.  Wave-uniform call.
template <typename E>
__device__ __forceinline__ void step_block(const StepParams& S, int cid, unsigned long long word, const double* tab) {
    const Params& P = S.p;
    const int lane = threadIdx.x & 63;
    const int NB = P.nblocks;
    const int b = cid / NB;
    const int j = cid - b * NB;
    const int kind = static_cast<int>((word >> 30) & 3u);
    const int row = static_cast<int>(word & 0x3fffffffu);
    BlockRec* recs = P.recs + (size_t)b * NB;
    DrawRow<E> d;
    const bool work = (kind == kDrawResidual || kind == kDrawBonus) &&
                      row < P.total_draft + P.batch && row - b >= 0;
    if (work) {
        const DrawParams* dp = &S.dparams[b];
        init_draw_row<E>(d, P, kind, row, row - b, ld_coherent(&dp->pos), ld_coherent(&dp->v),
                         ld_coherent(&dp->m), ld_coherent(&dp->z32), P.temperature[b]);
        draw_blocks<E>(d, P.vocab, recs, j, 1, j + 1, tab);
    }
    wait_stores();
    int last = 0;
    if (lane == 0) {
        last = (arrive(&P.draw_cnt[b]) == static_cast<uint32_t>(NB - 1));
        if (last) reset_counter(&P.draw_cnt[b]);
    }
    if (rdlane(last, 0) && work) {
        const int y = draw_select_wave<E>(d, P.vocab, NB, recs, tab, P.err);
        if (lane == 0 && d.pos >= 0 && d.pos <= P.gamma)
            st_coherent(&P.out_tokens[(size_t)b * (P.gamma + 1) + d.pos], y);
    }
}

// Row waves: pieces in position-major order as one continuous stream.  Three
// batches (six vectors per lane) are always in flight: while the current
// piece's batch e is consumed, batch e + 3 is issued, which for the piece's
// last three batches is the next piece's first three.
template <typename E>
__device__ __forceinline__ void row_wave(const StepParams& S, int w, int R, const double* tab, int* defer) {
    const Params& P = S.p;
    const int lane = threadIdx.x & 63;
    // candidates w, w + R, ... with their request words loaded two ahead
    Cand c0 = cand_load(S, w);
    Cand c1 = cand_load(S, w + R);
    int nd = 0, qd = 0;                       // deferred pieces: count, next
    // picks the next item to stream (deferring pieces of resolved requests) and
    // issues its small loads; it.j = -1 when there is none
    auto pick = [&](Item& it) {
        while (c0.j < S.items) {
            const Cand c = c0;
            c0 = c1;
            c1 = cand_load(S, c0.j + R);
            if (!item_coords(S, c.j, c.o0, c.o1, it)) continue;
            const int k = resolved_at(unpack_state(c.st), it.gb);
            if (k >= 0 && k < it.i && nd < kMaxDeferred) {
                if (lane == 0) defer[nd] = c.j;
                ++nd;
                continue;
            }
            item_issue<E>(S, it);
            return;
        }
        while (qd < nd) {
            __syncthreads();
            const int j = defer[qd++];
            int o0 = 0, o1 = 0;
            if (P.offsets) {
                const int b = (j / S.pieces) % P.batch;
                o0 = P.offsets[b];
                o1 = P.offsets[b + 1];
            }
            if (!item_coords(S, j, o0, o1, it)) continue;
            item_issue<E>(S, it);
            return;
        }
        it.j = -1;
    };
    Item cur, nxt;
    pick(cur);
    if (cur.j < 0) return;
    pick(nxt);
    v4u R0[kStepBatch], R1[kStepBatch], R2[kStepBatch];
    issue_batch(cur, 0, R0);
    issue_batch(cur, 1, R1);
    issue_batch(cur, 2, R2);
    Arrival arr;
    arr.valid = false;
    while (cur.j >= 0) {
        const float T = cur.T;
        const bool greedy = !(T > 0.0f);
        const float c = greedy ? 0.0f : static_cast<float>(kLog2e / static_cast<double>(T));
        // piece 0 of a draft row gathers the drafted token's logit and q; every
        // lane loads (an in-range element when it has nothing to gather), so
        // no branch makes the compiler wait for the loads in flight
        const bool gather = cur.xd >= 0 && cur.xd < P.vocab && !greedy;
        const long tcur = (long)cur.d0 + cur.b + cur.i;
        const int xg = gather ? cur.xd : 0;
        const uint32_t lx_bits = E::bits1(static_cast<const typename E::T*>(P.logits) + (size_t)tcur * P.vocab, xg);
        const float* qp = gather ? P.q + (size_t)(cur.d0 + cur.i) * P.vocab + xg : P.uniforms;
        const float qx_raw = *qp;
        PieceAcc acc;
        acc.mt = -INFINITY;
        acc.bi = 0x7fffffff;
        acc.st = 0.0;
        // with no next piece, the last three issues re-read this piece (never consumed)
        const Item& nx = (nxt.j >= 0) ? nxt : cur;
        consume_batch<E>(cur, 0, R0, greedy, c, tab, acc);
        issue_batch(cur, 3, R0);
        consume_batch<E>(cur, 1, R1, greedy, c, tab, acc);
        issue_batch(cur, 4, R1);
        consume_batch<E>(cur, 2, R2, greedy, c, tab, acc);
        issue_batch(cur, 5, R2);
        // the previous piece's arrival has had a few batches' worth of time to return
        if (arr.valid) finish_arrival<E>(S, arr, tab);
        arr.valid = false;
        consume_batch<E>(cur, 3, R0, greedy, c, tab, acc);
        issue_batch(nx, 0, R0);
        consume_batch<E>(cur, 4, R1, greedy, c, tab, acc);
        issue_batch(nx, 1, R1);
        consume_batch<E>(cur, 5, R2, greedy, c, tab, acc);
        issue_batch(nx, 2, R2);
        const float lx = gather ? E::from_bits(lx_bits) : 0.0f;
        const float qx = gather ? qx_raw : 0.0f;
        arr = item_finish<E>(S, cur, greedy, c, acc, lx, qx, tab);
        const bool more = nxt.j >= 0;
        cur = nxt;
        if (more) pick(nxt);
    }
    if (arr.valid) finish_arrival<E>(S, arr, tab);
}

// Draw waves: draw block q of wave dw is block dw + q * D of the call
// (request-major), worked on once its request is published.
template <typename E>
__device__ __forceinline__ void draw_wave(const StepParams& S, int dw, int D, const double* tab) {
    const Params& P = S.p;
    const int lane = threadIdx.x & 63;
    const int NB = P.nblocks;
    const int own = dw + lane * D;
    unsigned long long pending = __ballot(lane < kMaxOwnBlocks && own < P.batch * NB);
    const int own_req = own / NB;
    int spins = 0;
    while (pending != 0ull) {
        unsigned long long wd = 0ull;
        if ((pending >> lane) & 1ull) wd = ld_coherent(&S.words[own_req]);
        unsigned long long ready =
            __ballot(((pending >> lane) & 1ull) && static_cast<uint32_t>(wd >> 32) == S.epoch);
        if (ready == 0ull) {
            // a publication can only be missing when a row was rejected for
            // inconsistent offsets; stop waiting as soon as that is flagged, and
            // count the abandoned blocks as arrived (no draw) so counters stay balanced
            if (++spins >= kSpinLimit || (ld_coherent(P.err) & kErrOffsets) != 0u) {
                if (lane == 0) flag_error(P.err, spins >= kSpinLimit ? (kErrOffsets | kErrStalled) : kErrOffsets);
                wd = static_cast<unsigned long long>(S.epoch) << 32;
                ready = pending;
            } else {
                __builtin_amdgcn_s_sleep(2);
                continue;
            }
        }
        pending &= ~ready;
        while (ready != 0ull) {
            const int q = __ffsll(static_cast<long long>(ready)) - 1;
            ready &= ready - 1ull;
            step_block<E>(S, rdlane(own, q), rdlane_u64(wd, q), tab);
        }
    }
}

// Workgroups [0, row_waves) are row waves, the rest draw waves.
template <typename E>
__global__ __launch_bounds__(kStepLanes, 3) void step_kernel(StepParams S) {
    __shared__ double tab[64];
    __shared__ int defer[kMaxDeferred];
    const int lane = threadIdx.x;
    const int w = blockIdx.x;
    tab[lane] = kExp2Table[lane];
    __syncthreads();
    if (w < S.row_waves) row_wave<E>(S, w, S.row_waves, tab, defer);
    else draw_wave<E>(S, w - S.row_waves, static_cast<int>(gridDim.x) - S.row_waves, tab);
}

}  // namespace sv
