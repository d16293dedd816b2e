// zero1_noalloc.hip -- neox_zero1_step_noalloc: one step of the ZeRO-1 mixed-precision
// Adam update with no handle and no device allocation, for callers that cannot allocate
// device memory (tight serving loops, harnesses that forbid hipMalloc).  It uploads its
// tables and reads the state back with a stream synchronization, so it is not a call to
// record inside a HIP graph capture.
//
// Everything the step's kernels need besides the caller's arrays -- the device state
// block, the norm pass's per-block partial sums and the work tables -- lives in one
// file-scope device array, `scratch`, of a fixed size.  Each device holds its own copy
// for the life of the process.  The kernels and their launch shapes are the ones
// neox_zero1_step runs, so both give the same bits for the same inputs.
#include "neox_zero1.h"
#include "zero1_internal.h"

#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

using namespace nz1;

// The scratch array.  In host code its name is only a stand-in for the symbol: host code
// uses the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[NEOX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    int rc = NEOX_OK;            // result of the set-up below (kept for later calls)
    unsigned char* ptr = nullptr;
    std::mutex busy;             // calls on one device run one at a time
};
DeviceScratch g_dev[kMaxDevices];

// Once per device, with that device current: the device address of `scratch`.
int device_scratch(int device, unsigned char** out) {
    DeviceScratch& d = g_dev[device];
    std::call_once(d.once, [&d]() {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) {
            d.rc = set_hip_error(e, "hipGetSymbolAddress(scratch)");
            return;
        }
        d.ptr = static_cast<unsigned char*>(p);
    });
    if (d.rc != NEOX_OK) return set_error(d.rc, "scratch set-up failed on device %d", device);
    *out = d.ptr;
    return NEOX_OK;
}

// Byte offsets of the regions inside scratch, each 256-byte aligned.
struct Layout {
    size_t state = 0, partial = 0, norm_table = 0, table = 0, words = 0, changes = 0, end = 0;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" int neox_zero1_step_noalloc(const neox_zero1_config* cfg, const neox_segment* segs,
                                       uint64_t nseg, neox_scaler_state_t* state, float lr,
                                       void* hip_stream) {
    if (!cfg || !state) return set_error(NEOX_EINVAL, "null argument");
    if (!std::isfinite(lr)) return set_error(NEOX_EINVAL, "lr %g is not finite", (double)lr);
    if (cfg->segment_norms)
        return set_error(NEOX_EINVAL, "segment_norms needs a handle (neox_zero1_create)");
    if (!(std::isfinite(state->loss_scale) && state->loss_scale > 0.0f))
        return set_error(NEOX_EINVAL, "loss_scale %g", (double)state->loss_scale);
    if (state->good_steps < 0 || state->step < 0 || state->skipped_total < 0 ||
        state->consecutive_overflows < 0)
        return set_error(NEOX_EINVAL, "negative counter in the scaler state");

    Plan plan;
    int rc = make_plan(cfg, segs, nseg, plan);
    if (rc) return rc;
    const uint32_t nnorm = (uint32_t)plan.norm_table.size();
    uint32_t nb = cfg->norm_blocks ? cfg->norm_blocks : nnorm;
    if (nb > nnorm) nb = nnorm;
    if (nb == 0) nb = 1;

    Layout L;
    L.state = 0;
    L.partial = round256(2 * sizeof(DevState));   // the state block and its snapshot
    L.norm_table = round256(L.partial + (size_t)nb * sizeof(double));
    L.table = round256(L.norm_table + plan.norm_table.size() * sizeof(Chunk));
    size_t end = L.table;
    if (plan.flat) {
        L.words = L.table;
        L.changes = round256(L.words + plan.tile_word.size() * sizeof(uint32_t));
        end = L.changes + (plan.change.size() + 1) * sizeof(uint32_t);
    } else {
        end = L.table + plan.table.size() * sizeof(Chunk);
    }
    L.end = round256(end);
    if (L.end > (size_t)NEOX_NOALLOC_SCRATCH_BYTES)
        return set_error(NEOX_EINVAL,
                         "%llu elements in %llu segments need %zu bytes of scratch; the maximum "
                         "is %d (use neox_zero1_create)",
                         (unsigned long long)plan.numel, (unsigned long long)nseg, L.end,
                         NEOX_NOALLOC_SCRATCH_BYTES);

    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
    if (device < 0 || device >= kMaxDevices)
        return set_error(NEOX_EINVAL, "device %d: at most %d devices", device, kMaxDevices);
    unsigned char* base = nullptr;
    rc = device_scratch(device, &base);
    if (rc) return rc;
    LdsReserve lds;
    rc = lds_reserve(device, cfg->optimizer,
                     plan.flat ? (uint64_t)plan.tile_word.size() - 1 : (uint64_t)plan.table.size(),
                     &lds);
    if (rc) return rc;

    // Host image of everything the kernels read from scratch, uploaded in one copy.
    std::vector<unsigned char> img;
    try {
        img.assign(L.end, 0);
    } catch (const std::exception&) {
        return set_error(NEOX_ENOMEM, "host allocation of the upload image");
    }
    const DevState st0 = initial_state(*cfg, state->loss_scale, state->good_steps, state->step,
                                       state->skipped_total, state->consecutive_overflows);
    std::memcpy(img.data() + L.state, &st0, sizeof st0);
    std::memcpy(img.data() + L.norm_table, plan.norm_table.data(), plan.norm_table.size() * sizeof(Chunk));
    if (plan.flat) {
        std::memcpy(img.data() + L.words, plan.tile_word.data(), plan.tile_word.size() * sizeof(uint32_t));
        if (!plan.change.empty())
            std::memcpy(img.data() + L.changes, plan.change.data(), plan.change.size() * sizeof(uint32_t));
    } else {
        std::memcpy(img.data() + L.table, plan.table.data(), plan.table.size() * sizeof(Chunk));
    }

    DevState* d_state = reinterpret_cast<DevState*>(base + L.state);
    StepLaunch sl;
    sl.dtype = cfg->dtype;
    sl.optimizer = cfg->optimizer;
    sl.norm_nt = plan.numel > kNormCachedMax;
    sl.norm_big = plan.norm_big;
    sl.norm_chunks = reinterpret_cast<const Chunk*>(base + L.norm_table);
    sl.nnorm = nnorm;
    sl.norm_blocks = nb;
    sl.partial = reinterpret_cast<double*>(base + L.partial);
    sl.st = d_state;
    sl.snap = d_state + 1;
    sl.fused = kUpdateDecides && nb <= kFuseMaxParts;
    sl.fin = finalize_args(*cfg);
    sl.upd = update_args(*cfg);
    sl.lds = lds;
    sl.flat = plan.flat;
    if (plan.flat) {
        FlatSpan& sp = sl.span;
        sp.grad = static_cast<const uint16_t*>(segs[0].grad);
        sp.half = static_cast<uint16_t*>(segs[0].half);
        sp.master = segs[0].master;
        sp.m = segs[0].exp_avg;
        sp.v = cfg->optimizer == NEOX_OPT_ADAMW ? segs[0].exp_avg_sq : nullptr;
        sp.n = plan.numel;
        sp.tile_word = reinterpret_cast<const uint32_t*>(base + L.words);
        sp.change = reinterpret_cast<const uint32_t*>(base + L.changes);
        sp.ntiles = (uint32_t)(plan.tile_word.size() - 1);
    } else {
        sl.chunks = reinterpret_cast<const Chunk*>(base + L.table);
        sl.nchunks = (uint32_t)plan.table.size();
    }
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);

    DeviceScratch& d = g_dev[device];
    std::lock_guard<std::mutex> hold(d.busy);
    // Every region the kernels read is written by this copy (the snapshot by the norm
    // pass, the partials by the norm pass, both before they are read): nothing depends on
    // what an earlier call left in scratch.
    e = hipMemcpyAsync(base, img.data(), L.end, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = enqueue_step(sl, lr, stream, nullptr);
    DevState st{};
    if (e == hipSuccess) e = hipMemcpyAsync(&st, d_state, sizeof st, hipMemcpyDeviceToHost, stream);
    // the upload image and the state copy must outlive the stream's use of them
    const hipError_t es = hipStreamSynchronize(stream);
    if (e != hipSuccess) return set_hip_error(e, "step_noalloc launch");
    if (es != hipSuccess) return set_hip_error(es, "hipStreamSynchronize");
    state->loss_scale = st.loss_scale;
    state->good_steps = st.good_steps;
    state->step = st.step;
    state->skipped_total = st.skipped_total;
    state->consecutive_overflows = st.consecutive_overflows;
    state->last_skipped = st.last_skipped;
    state->last_grad_norm = st.last_grad_norm;
    state->last_clip_coef = st.last_clip_coef;
    state->last_sumsq = st.last_sumsq;
    state->device_loss_scale = nullptr;
    return NEOX_OK;
}
