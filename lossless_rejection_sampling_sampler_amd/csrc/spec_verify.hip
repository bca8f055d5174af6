// Host side of the speculative-decoding verifier: the C ABI declared in
// include/spec_verify.h (context, argument checks, scratch, launches).
//
// Method: the spec-decoding page at dpshk.com/news/5598276, sections 3.1-3.2,
// 5.2-5.4 and 8 (see the header for the operation and the readings).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "spec_verify.h"
#include "sv_device.h"

namespace {

constexpr int kRowVecsPerThread = 8;    // target 16-byte vectors per thread per row split
constexpr int kProfileRing = 2048;      // calls between forced event folds
constexpr int kDrawBlocksPerWave = 2;   // draw kernel: blocks per wave in straight-line code
constexpr int kDrawPerCU = 4;           // draw kernel (at most two blocks per wave): workgroups per CU aimed at
constexpr int kDrawLoopPerCU = 3;       // draw kernel taking pairs of blocks in a loop: what it holds per CU

struct Geometry {
    int splits;          // split rows kernel: workgroups per row
    int nblocks;         // draw blocks per row
};

Geometry geometry_for(int vocab, int dtype) {
    const int esize = (dtype == SV_BF16) ? 2 : 4;
    const long nvec = ((long)vocab * esize + 15) / 16;
    long s = (nvec + (long)sv::kThreads * kRowVecsPerThread - 1) / ((long)sv::kThreads * kRowVecsPerThread);
    s = std::max(1L, std::min(s, (long)sv::kMaxPieces));
    Geometry g;
    g.splits = static_cast<int>(s);
    g.nblocks = (vocab + sv::kBlockElems - 1) / sv::kBlockElems;
    return g;
}

// Workgroups for the flat rows stream: all resident at
// once, at least one batch of loads per thread or else one workgroup per row (a
// small call is latency-bound: its rows then stream side by side), and no row
// cut into more than kMaxPieces pieces.
int flat_workgroups(long nv, long vpr, int resident) {
    const long rows = vpr > 0 ? nv / vpr : 1;
    long g = std::min<long>(resident, std::max<long>(rows, nv / ((long)sv::kThreads * sv::kRowUnroll)));
    while (g > 1) {
        const long lmin = nv / g;
        const long pmax = (vpr + lmin - 1) / lmin + 1;
        if (pmax <= sv::kMaxPieces) break;
        --g;
    }
    return static_cast<int>(std::max<long>(1, g));
}

// Rows kernel then draw kernel on `stream`.  ev, when given, holds four events
// that the dispatches themselves stamp: rows start / end, draw start / end (the
// kernels' own execution, without the gap between dispatches).
// The draw kernel's variant: kLoop (waves take pairs of blocks in a loop),
// kSplit (one workgroup per block, its waves on the block's sub-blocks), or
// neither (at most two blocks per wave).
template <typename E, bool kLoop, bool kSplit>
void launch_draw(dim3 g2, dim3 blk, const sv::Params& P, hipStream_t stream, const hipEvent_t* ev) {
    if (ev) hipExtLaunchKernelGGL((sv::draw_kernel<E, kLoop, kSplit>), g2, blk, 0, stream, ev[2], ev[3], 0, P);
    else hipLaunchKernelGGL((sv::draw_kernel<E, kLoop, kSplit>), g2, blk, 0, stream, P);
}

// Rows kernel then draw kernel on `stream`.  ev, when given, holds four events
// that the dispatches themselves stamp: rows start / end, draw start / end (the
// kernels' own execution, without the gap between dispatches).  draw: 0 pairs
// of blocks at most per wave, 1 pairs in a loop, 2 split blocks.
template <typename E>
int launch_rows_draw(bool aligned, int draw, long grid1, long grid2, const sv::Params& P, hipStream_t stream,
                     const hipEvent_t* ev) {
    const dim3 g1((unsigned)grid1), g2((unsigned)grid2), blk(sv::kThreads);
    if (!ev) {
        if (aligned) hipLaunchKernelGGL(sv::rows_flat_kernel<E>, g1, blk, 0, stream, P);
        else hipLaunchKernelGGL(sv::rows_split_kernel<E>, g1, blk, 0, stream, P);
    } else if (aligned) {
        hipExtLaunchKernelGGL(sv::rows_flat_kernel<E>, g1, blk, 0, stream, ev[0], ev[1], 0, P);
    } else {
        hipExtLaunchKernelGGL(sv::rows_split_kernel<E>, g1, blk, 0, stream, ev[0], ev[1], 0, P);
    }
    if (draw == 1) launch_draw<E, true, false>(g2, blk, P, stream, ev);
    else if (draw == 2) launch_draw<E, false, true>(g2, blk, P, stream, ev);
    else launch_draw<E, false, false>(g2, blk, P, stream, ev);
    return SV_OK;
}

static_assert(SV_MAX_GAMMA + 1 <= sv::kMaxReqRows, "a request's rows fit the draw kernel's resolve");

// Scratch the kernels of one call use (device memory) and the host-mapped
// contract word (may be null).
struct Scratch {
    sv::Piece* parts;
    sv::RowStat* rows;
    sv::BlockRec* recs;
    uint32_t* draw_cnt;
    uint32_t* err;
    uint32_t* err_host;
};

// Host-visible argument checks (nothing is enqueued unless SV_OK); *qmode
// receives how q is given.
int check_args(int max_batch, int max_gamma, int vocab, int dtype, const sv_args* a, int* qmode) {
    if (a->batch < 0 || a->gamma < 0 || a->total_draft < 0) return SV_ERR_INVALID_ARG;
    *qmode = sv::kQDense;
    if (a->batch == 0) return SV_OK;
    if (a->batch > max_batch || a->gamma > max_gamma) return SV_ERR_CAPACITY;
    if (a->vocab != vocab) return SV_ERR_INVALID_ARG;   // one vocabulary for draft and target
    if ((long)a->total_draft > (long)a->batch * a->gamma) return SV_ERR_INVALID_ARG;
    if (!a->draft_offsets && a->total_draft != a->batch * a->gamma) return SV_ERR_INVALID_ARG;
    if (!a->target_logits || !a->temperature || !a->uniforms || !a->out_tokens || !a->out_num_accepted)
        return SV_ERR_INVALID_ARG;
    if (a->total_draft > 0 && !a->draft_ids) return SV_ERR_INVALID_ARG;
    // q: dense rows, sparse (id, prob) entries, or point masses at the drafted tokens
    if (!a->draft_probs) {
        if (a->draft_topk < 0 || a->draft_topk > SV_MAX_TOPK) return SV_ERR_INVALID_ARG;
        *qmode = a->draft_topk > 0 ? sv::kQSparse : sv::kQPoint;
        if (*qmode == sv::kQSparse && a->total_draft > 0 && (!a->draft_topk_ids || !a->draft_topk_probs))
            return SV_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(a->draft_topk_ids) % 4 || reinterpret_cast<uintptr_t>(a->draft_topk_probs) % 4)
            return SV_ERR_INVALID_ARG;
    }
    if (reinterpret_cast<uintptr_t>(a->stats) % 4) return SV_ERR_INVALID_ARG;
    const size_t esize = (dtype == SV_BF16) ? 2 : 4;
    if (reinterpret_cast<uintptr_t>(a->target_logits) % esize) return SV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(a->draft_probs) % 4 || reinterpret_cast<uintptr_t>(a->draft_ids) % 4)
        return SV_ERR_INVALID_ARG;
    return SV_OK;
}

// Enqueues the rows kernel and the draw kernel of one checked call (batch > 0)
// on `stream`; `ev` (null, or four events) times the two dispatches.  *schedule
// receives the SV_SCHEDULE_* launched.
int enqueue(const Geometry& geo, int resident_flat, int cus, int resident_draw, int dtype, const Scratch& sc,
            const sv_args* a, int qmode, hipStream_t stream, const hipEvent_t* ev, int* schedule) {
    const size_t esize = (dtype == SV_BF16) ? 2 : 4;
    sv::Params P;
    P.logits = a->target_logits;
    P.q = a->draft_probs;
    P.ids = a->draft_ids;
    P.temperature = a->temperature;
    P.uniforms = a->uniforms;
    P.offsets = a->draft_offsets;
    P.out_tokens = a->out_tokens;
    P.out_num = a->out_num_accepted;
    P.diag_m = a->diag_row_max;
    P.diag_z = a->diag_row_norm;
    P.diag_r = a->diag_ratio;
    P.qmode = qmode;
    P.topk = qmode == sv::kQSparse ? a->draft_topk : 0;
    P.topk_ids = qmode == sv::kQSparse ? a->draft_topk_ids : nullptr;
    P.topk_probs = qmode == sv::kQSparse ? a->draft_topk_probs : nullptr;
    P.stats = a->stats;
    P.batch = a->batch;
    P.gamma = a->gamma;
    P.total_draft = a->total_draft;
    P.vocab = a->vocab;
    P.splits = geo.splits;
    P.nblocks = geo.nblocks;
    // draw workgroups per request: four per CU over the call (one resident
    // round; measured 23.1 against 23.8 us for three on B = 64, V = 151936)
    // where that keeps between one and kDrawBlocksPerWave blocks per wave.  A
    // call with more draw rows than that round can hold at two blocks per wave
    // (B = 128 or 256 at V = 151936 / 128256) has its waves take pairs of
    // blocks in a loop, in one resident round at three workgroups per CU
    // (draw kernel, against a second round of workgroups: B = 128 T mix 32.1
    // against 34.5 us, B = 256 ragged 44.0 against 45.2, B = 256 top-50 q in
    // dense rows 47.0 against 52.1; four per CU was faster on some of these and
    // slower on others)
    const int c_min = std::max(1, (geo.nblocks + sv::kWaves * kDrawBlocksPerWave - 1) /
                                      (sv::kWaves * kDrawBlocksPerWave));
    const int c_max = std::max(1, (geo.nblocks + sv::kWaves - 1) / sv::kWaves);
    const int c_fit = kDrawPerCU * cus / a->batch;
    const bool draw_loop = c_fit < c_min;
    const int c_fit_loop = kDrawLoopPerCU * cus / a->batch;
    // a call whose blocks all fit one resident round as separate workgroups
    // (small batches and vocabularies: latency-bound) gives every block its own
    // workgroup, the block's four sub-blocks to its four waves
    const bool split = (long)a->batch * geo.nblocks <= (long)resident_draw;
    const int C = split ? geo.nblocks
                        : (draw_loop ? std::max(1, c_fit_loop) : std::max(c_min, std::min(c_max, c_fit)));
    P.draw_wgs = C;
    P.parts = sc.parts;
    P.rows = sc.rows;
    P.recs = sc.recs;
    P.draw_cnt = sc.draw_cnt;
    P.err = sc.err;
    P.err_host = sc.err_host;

    const long rows = (long)a->total_draft + a->batch;
    // rows start on 16-byte boundaries: stream the flattened rows in equal ranges
    P.flat_vpr = (long)a->vocab * (long)esize / 16;
    P.flat_nv = rows * P.flat_vpr;
    // (the flat kernel's range arithmetic needs flat_nv * grid below 2^52: far
    // beyond any call that fits in device memory, but checked)
    const bool aligned = (reinterpret_cast<uintptr_t>(a->target_logits) % 16 == 0) &&
                         (((long)a->vocab * (long)esize) % 16 == 0) &&
                         static_cast<double>(P.flat_nv) * resident_flat < 4.5e15;
    // rows are streamed without any hand-off between workgroups (flattened
    // ranges for 16-byte aligned rows, per-row splits otherwise) and every
    // request is resolved by its draw workgroups
    const long grid1 = aligned ? flat_workgroups(P.flat_nv, P.flat_vpr, resident_flat) : rows * P.splits;
    const long grid2 = (long)a->batch * C;
    P.rows_grid = static_cast<int>(grid1);
    if (aligned) {
        const long lmin = P.flat_nv / grid1;       // shortest range
        P.max_pieces = static_cast<int>(std::min<long>(sv::kMaxPieces, (P.flat_vpr + lmin - 1) / lmin + 1));
    } else {
        P.max_pieces = P.splits;
    }
    P.flat_inv_nv = 1.0 / static_cast<double>(P.flat_nv);
    P.flat_inv_vpr = 1.0 / static_cast<double>(P.flat_vpr);
    P.flat_inv_grid = 1.0 / static_cast<double>(grid1);
    P.draw_cmajor = grid2 <= resident_draw ? 1 : 0;
    const int st = (dtype == SV_BF16)
                       ? launch_rows_draw<sv::BF16>(aligned, split ? 2 : (draw_loop ? 1 : 0), grid1, grid2, P, stream, ev)
                       : launch_rows_draw<sv::F32>(aligned, split ? 2 : (draw_loop ? 1 : 0), grid1, grid2, P, stream, ev);
    if (st != SV_OK) return st;
    *schedule = aligned ? SV_SCHEDULE_FLAT : SV_SCHEDULE_SPLIT;
    return SV_OK;
}

}  // namespace

struct sv_ctx {
    int device = 0;
    sv_config cfg{};
    Geometry geo{};
    int max_rows = 0;
    int resident_flat = 0;     // rows-flat workgroups resident at once on the device
    int cus = 0;               // compute units of the device
    int resident_draw = 0;     // draw workgroups resident at once
    int last_schedule = SV_SCHEDULE_NONE;
    // device scratch (one allocation)
    void* scratch = nullptr;
    sv::Piece* parts = nullptr;
    sv::RowStat* rows = nullptr;
    sv::BlockRec* recs = nullptr;
    uint32_t* draw_cnt = nullptr;
    uint32_t* err = nullptr;
    // host-mapped pinned word the kernels set on a contract violation (checked by run)
    uint32_t* err_host = nullptr;
    uint32_t* err_host_dev = nullptr;   // its device-side address
    uint32_t* err_read = nullptr;       // pinned staging word for spec_verify_device_errors
    hipStream_t aux = nullptr;          // internal non-blocking stream: clears and reads of the error word
    hipStream_t last_stream = nullptr;  // stream of the last eagerly enqueued call
    bool have_last = false;
    // profiling
    std::vector<hipEvent_t> events;    // 4 per call: rows start / end, draw start / end
    int prof_n = 0;
    double prof_rows_ms = 0.0, prof_draw_ms = 0.0;
    int prof_calls = 0;
};

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
constexpr size_t align_up_c(size_t x, size_t a) { return (x + a - 1) / a * a; }

int fold_profile(sv_ctx* ctx) {
    if (ctx->prof_n == 0) return SV_OK;
    if (hipEventSynchronize(ctx->events[4 * (ctx->prof_n - 1) + 3]) != hipSuccess) return SV_ERR_DEVICE;
    for (int i = 0; i < ctx->prof_n; ++i) {
        float a = 0.f, b = 0.f;
        if (hipEventElapsedTime(&a, ctx->events[4 * i], ctx->events[4 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&b, ctx->events[4 * i + 2], ctx->events[4 * i + 3]) != hipSuccess)
            return SV_ERR_DEVICE;
        ctx->prof_rows_ms += a;
        ctx->prof_draw_ms += b;
    }
    ctx->prof_calls += ctx->prof_n;
    ctx->prof_n = 0;
    return SV_OK;
}

void free_ctx(sv_ctx* ctx) {
    if (!ctx) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(ctx->device);
    for (hipEvent_t e : ctx->events) (void)hipEventDestroy(e);
    if (ctx->aux) (void)hipStreamDestroy(ctx->aux);
    if (ctx->err_host) (void)hipHostFree(ctx->err_host);
    if (ctx->err_read) (void)hipHostFree(ctx->err_read);
    if (ctx->scratch) (void)hipFree(ctx->scratch);
    (void)hipSetDevice(prev);
    delete ctx;
}

// Waits for the stream of the context's last eagerly launched call and for the
// context's internal stream; no other stream is waited for.
int wait_context(sv_ctx* ctx) {
    if (ctx->have_last && hipStreamSynchronize(ctx->last_stream) != hipSuccess) return SV_ERR_DEVICE;
    if (ctx->aux && hipStreamSynchronize(ctx->aux) != hipSuccess) return SV_ERR_DEVICE;
    return SV_OK;
}

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) (void)hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (prev >= 0 && cur != prev) (void)hipSetDevice(prev);
    }
};

}  // namespace

// ----------------------------------------------------------------- entry point without allocation
// spec_verify_run_static keeps its scratch in this file-scope device array:
// each GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` is only a stand-in for the symbol; the device address is
// looked up once per device with hipGetSymbolAddress and used everywhere.
namespace {

constexpr size_t kStaticRows = SV_STATIC_MAX_ROWS;
constexpr size_t kStaticBatch = SV_STATIC_MAX_BATCH;
constexpr size_t kOffParts = 0;
constexpr size_t kOffRows = align_up_c(kOffParts + kStaticRows * sv::kMaxPieces * sizeof(sv::Piece), 256);
constexpr size_t kOffRecs = align_up_c(kOffRows + kStaticRows * sizeof(sv::RowStat), 256);
constexpr size_t kStaticRecs = SV_STATIC_MAX_DRAW_BLOCKS;   // draw block records (batch times blocks per row) at most
constexpr size_t kOffCnt = align_up_c(kOffRecs + kStaticRecs * sizeof(sv::BlockRec), 256);
constexpr size_t kStaticBytes = align_up_c(kOffCnt + (kStaticBatch + 1) * sizeof(uint32_t), 256);
static_assert(kStaticBytes <= SV_STATIC_SCRATCH_BYTES, "the static scratch holds its layout");

static __device__ __align__(256) unsigned char scratch[SV_STATIC_SCRATCH_BYTES];

constexpr int kStaticDevices = 64;
struct StaticDevice {
    bool ready = false;
    unsigned char* base = nullptr;     // device address of this device's `scratch`
    int cus = 0, resident_flat = 0, resident_draw = 0;
};
StaticDevice g_static[kStaticDevices];
std::mutex g_static_mu;

// Set-up on the current device, once: the scratch array's device address and
// the occupancy figures the launch geometry uses.
int static_device(int dev, StaticDevice** out) {
    if (dev < 0 || dev >= kStaticDevices) return SV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticDevice& sd = g_static[dev];
    if (!sd.ready) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return SV_ERR_DEVICE;
        }
        int cus = 0, per_cu = 0, per_draw = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sv::rows_flat_kernel<sv::BF16>, sv::kThreads, 0) !=
                hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_draw, sv::draw_kernel<sv::BF16, false>, sv::kThreads, 0) !=
                hipSuccess) {
            (void)hipGetLastError();
            return SV_ERR_DEVICE;
        }
        sd.base = static_cast<unsigned char*>(ptr);
        sd.cus = std::max(1, cus);
        sd.resident_flat = sd.cus * std::min(3, std::max(1, per_cu));
        sd.resident_draw = per_draw > 0 ? sd.cus * per_draw : 3 * sd.cus;
        sd.ready = true;
    }
    *out = &sd;
    return SV_OK;
}

}  // namespace

extern "C" {

const char* spec_verify_status_string(int status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_ERR_INVALID_ARG: return "invalid argument";
        case SV_ERR_OUT_OF_MEMORY: return "out of device memory";
        case SV_ERR_DEVICE: return "HIP device error";
        case SV_ERR_UNSUPPORTED: return "unsupported configuration";
        case SV_ERR_CAPACITY: return "exceeds the context's limits";
        case SV_ERR_DEVICE_CONTRACT: return "an earlier call broke the device-side contract";
        default: return "unknown status";
    }
}

int spec_verify_create(const sv_config* cfg, int device, sv_ctx** out) {
    if (!out) return SV_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg) return SV_ERR_INVALID_ARG;
    if (cfg->max_batch < 1 || cfg->max_gamma < 0 || cfg->max_gamma > SV_MAX_GAMMA || cfg->vocab < 1)
        return SV_ERR_INVALID_ARG;
    if (cfg->logits_dtype != SV_F32 && cfg->logits_dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
    if ((long)cfg->vocab > (long)sv::kMaxVocab) return SV_ERR_UNSUPPORTED;
    // row indices are 32-bit: max_batch * (max_gamma + 1) target rows must fit
    if ((long)cfg->max_batch * ((long)cfg->max_gamma + 1) > (long)INT32_MAX) return SV_ERR_UNSUPPORTED;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return SV_ERR_DEVICE;

    sv_ctx* ctx = new (std::nothrow) sv_ctx();
    if (!ctx) return SV_ERR_OUT_OF_MEMORY;
    ctx->device = device;
    ctx->cfg = *cfg;
    ctx->geo = geometry_for(cfg->vocab, cfg->logits_dtype);
    ctx->max_rows = cfg->max_batch * (cfg->max_gamma + 1);

    DeviceGuard guard(device);
    {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sv::rows_flat_kernel<sv::BF16>, sv::kThreads, 0) != hipSuccess) {
            delete ctx;
            return SV_ERR_DEVICE;
        }
        // at most three rows workgroups per CU: more make each CU's last one finish later
        ctx->resident_flat = std::max(1, cus * std::min(3, std::max(1, per_cu)));
        ctx->cus = std::max(1, cus);

        int per_draw = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_draw, sv::draw_kernel<sv::BF16, false>,
                                                         sv::kThreads, 0) == hipSuccess)
            ctx->resident_draw = cus * per_draw;
        if (ctx->resident_draw <= 0) ctx->resident_draw = 3 * std::max(1, cus);
        (void)hipGetLastError();
    }
    const size_t n_rows = (size_t)ctx->max_rows;
    const size_t n_b = (size_t)cfg->max_batch;
    size_t off = 0;
    const size_t o_parts = off; off = align_up(off + n_rows * sv::kMaxPieces * sizeof(sv::Piece), 256);
    const size_t o_rows = off;  off = align_up(off + n_rows * sizeof(sv::RowStat), 256);
    const size_t o_recs = off;  off = align_up(off + n_b * ctx->geo.nblocks * sizeof(sv::BlockRec), 256);
    const size_t o_cnt = off;   off = align_up(off + (n_b + 1) * sizeof(uint32_t), 256);
    const size_t total = off;
    if (hipMalloc(&ctx->scratch, total) != hipSuccess) {
        (void)hipGetLastError();
        delete ctx;
        return SV_ERR_OUT_OF_MEMORY;
    }
    char* base = static_cast<char*>(ctx->scratch);
    ctx->parts = reinterpret_cast<sv::Piece*>(base + o_parts);
    ctx->rows = reinterpret_cast<sv::RowStat*>(base + o_rows);
    ctx->recs = reinterpret_cast<sv::BlockRec*>(base + o_recs);
    ctx->draw_cnt = reinterpret_cast<uint32_t*>(base + o_cnt);
    ctx->err = ctx->draw_cnt + n_b;
    if (hipHostMalloc(reinterpret_cast<void**>(&ctx->err_host), sizeof(uint32_t),
                      hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess ||
        hipHostMalloc(reinterpret_cast<void**>(&ctx->err_read), sizeof(uint32_t), hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        free_ctx(ctx);
        return SV_ERR_OUT_OF_MEMORY;
    }
    *reinterpret_cast<volatile uint32_t*>(ctx->err_host) = 0u;
    if (hipHostGetDevicePointer(reinterpret_cast<void**>(&ctx->err_host_dev), ctx->err_host, 0) != hipSuccess ||
        hipStreamCreateWithFlags(&ctx->aux, hipStreamNonBlocking) != hipSuccess) {
        free_ctx(ctx);
        return SV_ERR_DEVICE;
    }
    if (hipMemsetAsync(ctx->scratch, 0, total, ctx->aux) != hipSuccess || hipStreamSynchronize(ctx->aux) != hipSuccess) {
        free_ctx(ctx);
        return SV_ERR_DEVICE;
    }
    if (cfg->flags & SV_FLAG_PROFILE) {
        ctx->events.resize(4 * kProfileRing, nullptr);
        for (auto& e : ctx->events) {
            if (hipEventCreate(&e) != hipSuccess) {
                e = nullptr;
                free_ctx(ctx);
                return SV_ERR_DEVICE;
            }
        }
    }
    *out = ctx;
    return SV_OK;
}

int spec_verify_destroy(sv_ctx* ctx) {
    if (!ctx) return SV_OK;
    {
        DeviceGuard guard(ctx->device);
        (void)wait_context(ctx);
    }
    free_ctx(ctx);
    return SV_OK;
}

int spec_verify_run(sv_ctx* ctx, const sv_args* a, void* stream_ptr) {
    if (!ctx || !a) return SV_ERR_INVALID_ARG;
    // a violation the device has reported (host-mapped word) blocks further calls
    // until spec_verify_device_errors clears it
    if (*reinterpret_cast<volatile uint32_t*>(ctx->err_host) != 0u) return SV_ERR_DEVICE_CONTRACT;
    const sv_config& cfg = ctx->cfg;
    int qmode = 0;
    const int st0 = check_args(cfg.max_batch, cfg.max_gamma, cfg.vocab, cfg.logits_dtype, a, &qmode);
    if (st0 != SV_OK) return st0;
    if (a->batch == 0) {
        ctx->last_schedule = SV_SCHEDULE_NONE;
        return SV_OK;
    }
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    DeviceGuard guard(ctx->device);

    Scratch sc;
    sc.parts = ctx->parts;
    sc.rows = ctx->rows;
    sc.recs = ctx->recs;
    sc.draw_cnt = ctx->draw_cnt;
    sc.err = ctx->err;
    sc.err_host = ctx->err_host_dev;

    const bool prof = (cfg.flags & SV_FLAG_PROFILE) != 0;
    if (prof && ctx->prof_n == kProfileRing) {
        const int st = fold_profile(ctx);
        if (st != SV_OK) return st;
    }
    const hipEvent_t* ev = prof ? &ctx->events[4 * ctx->prof_n] : nullptr;
    int schedule = SV_SCHEDULE_NONE;
    const int st = enqueue(ctx->geo, ctx->resident_flat, ctx->cus, ctx->resident_draw, cfg.logits_dtype, sc, a,
                           qmode, stream, ev, &schedule);
    if (st != SV_OK) return st;
    if (hipGetLastError() != hipSuccess) return SV_ERR_DEVICE;
    if (prof) ctx->prof_n++;
    // remember the stream this call was enqueued on (not while a graph is being
    // captured: a replay is waited for by the caller); an event per call would
    // add a marker between consecutive steps
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
        (void)hipGetLastError();
        cap = hipStreamCaptureStatusNone;
    }
    if (cap == hipStreamCaptureStatusNone) {
        ctx->last_stream = stream;
        ctx->have_last = true;
    }
    ctx->last_schedule = schedule;
    return SV_OK;
}

int spec_verify_last_schedule(const sv_ctx* ctx, int32_t* schedule) {
    if (!ctx || !schedule) return SV_ERR_INVALID_ARG;
    *schedule = ctx->last_schedule;
    return SV_OK;
}

int spec_verify_device_errors(sv_ctx* ctx, uint32_t* bits, int clear) {
    if (!ctx || !bits) return SV_ERR_INVALID_ARG;
    DeviceGuard guard(ctx->device);
    if (wait_context(ctx) != SV_OK) return SV_ERR_DEVICE;
    if (hipMemcpyAsync(ctx->err_read, ctx->err, sizeof(uint32_t), hipMemcpyDeviceToHost, ctx->aux) != hipSuccess ||
        hipStreamSynchronize(ctx->aux) != hipSuccess)
        return SV_ERR_DEVICE;
    *bits = *ctx->err_read | *reinterpret_cast<volatile uint32_t*>(ctx->err_host);
    if (clear) {
        if (hipMemsetAsync(ctx->err, 0, sizeof(uint32_t), ctx->aux) != hipSuccess ||
            hipStreamSynchronize(ctx->aux) != hipSuccess)
            return SV_ERR_DEVICE;
        *reinterpret_cast<volatile uint32_t*>(ctx->err_host) = 0u;
    }
    return SV_OK;
}

int spec_verify_profile_read(sv_ctx* ctx, double* rows_ms, double* draw_ms, int32_t* count) {
    if (!ctx || !rows_ms || !draw_ms || !count) return SV_ERR_INVALID_ARG;
    if (!(ctx->cfg.flags & SV_FLAG_PROFILE)) return SV_ERR_INVALID_ARG;
    DeviceGuard guard(ctx->device);
    const int st = fold_profile(ctx);
    if (st != SV_OK) return st;
    *rows_ms = ctx->prof_rows_ms;
    *draw_ms = ctx->prof_draw_ms;
    *count = ctx->prof_calls;
    ctx->prof_rows_ms = ctx->prof_draw_ms = 0.0;
    ctx->prof_calls = 0;
    return SV_OK;
}

int spec_verify_run_static(int logits_dtype, const sv_args* a, void* stream_ptr) {
    if (!a) return SV_ERR_INVALID_ARG;
    if (logits_dtype != SV_F32 && logits_dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
    if (a->vocab < 1) return SV_ERR_INVALID_ARG;
    if ((long)a->vocab > (long)sv::kMaxVocab) return SV_ERR_UNSUPPORTED;
    if (a->batch > SV_STATIC_MAX_BATCH || a->gamma > SV_MAX_GAMMA ||
        (long)a->total_draft + (long)a->batch > (long)SV_STATIC_MAX_ROWS ||
        (long)a->batch * ((a->vocab + sv::kBlockElems - 1) / sv::kBlockElems) > (long)kStaticRecs)
        return SV_ERR_CAPACITY;
    int qmode = 0;
    const int st0 = check_args(SV_STATIC_MAX_BATCH, SV_MAX_GAMMA, a->vocab, logits_dtype, a, &qmode);
    if (st0 != SV_OK) return st0;
    if (a->batch == 0) return SV_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_DEVICE;
    StaticDevice* sd = nullptr;
    const int st1 = static_device(dev, &sd);
    if (st1 != SV_OK) return st1;
    Scratch sc;
    sc.parts = reinterpret_cast<sv::Piece*>(sd->base + kOffParts);
    sc.rows = reinterpret_cast<sv::RowStat*>(sd->base + kOffRows);
    sc.recs = reinterpret_cast<sv::BlockRec*>(sd->base + kOffRecs);
    sc.draw_cnt = reinterpret_cast<uint32_t*>(sd->base + kOffCnt);
    sc.err = sc.draw_cnt + kStaticBatch;
    sc.err_host = nullptr;
    int schedule = SV_SCHEDULE_NONE;
    const int st = enqueue(geometry_for(a->vocab, logits_dtype), sd->resident_flat, sd->cus, sd->resident_draw,
                           logits_dtype, sc, a, qmode, static_cast<hipStream_t>(stream_ptr), nullptr, &schedule);
    if (st != SV_OK) return st;
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}

}  // extern "C"
