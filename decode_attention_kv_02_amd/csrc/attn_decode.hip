// attn_decode.hip -- C ABI, validation, workspace and launches of the
// split-KV decode-attention library (see include/attn_decode.h).
//
// Host-side validation rejects every bad shape, pointer, alignment and
// overlap before anything is enqueued, so the kernels only guard their own
// tails (the convention of tessl nn.rs: the wrappers reject out-of-bounds
// work on the host; flash_attn_decode validates dims, head_dim and capacity
// before encoding).  The slot table travels by value in the kernel arguments:
// no host-to-device copy, nothing to keep alive, nothing to synchronise.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/attn_decode.h"
#include "planner.hpp"
#include "attn_decode_kernels.hpp"
#include "attn_mfma_kernels.hpp"
#include "kv_append_kernels.hpp"
#include "fwht_kernels.hpp"

using namespace attn_decode_impl;

static_assert(ATTN_DECODE_MAX_SLOTS_PER_LAUNCH == kMaxSlotsPerLaunch, "slot table size");
static_assert(ATTN_DECODE_MAX_CHUNKS == kMaxChunks, "chunk bound");
static_assert(ATTN_DECODE_CHUNK_PER_CALL == kChunkPerCall, "per-call chunk floor");
static_assert(kSingleLaunchMaxChunks <= kMaxChunks, "single-launch merge bound");
static_assert(sizeof(LaunchArgsT<kSmallTableSlots>) <= 4096, "the small query table stays within 4 KiB of arguments");
// the large table: 18.5 KiB of kernel arguments, which ROCm copies whole (checked on MI355X up to 18 KiB)
static_assert(sizeof(LaunchArgsT<kMaxSlotsPerLaunch>) <= 20 * 1024, "large query table");
static_assert(sizeof(AppendArgs) <= 4096, "kernel arguments stay within 4 KiB");

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

// ------------------------------------------------------------ workspace cache

struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
    int64_t flag_bytes = 0;   // the flagged-pair region at the front; all zero between calls
};

std::mutex g_ws_mutex;
std::map<std::pair<int, void *>, Workspace> g_ws;  // keyed by (device, stream)
// Buffers a workspace outgrew, per device.  They stay allocated until
// attn_decode_release: a HIP graph captured earlier, work still queued, or
// another host thread may still hold their address.
std::vector<std::pair<int, void *>> g_retired;

// Returns the flagged-pair region (all zero) and the plain partials area of the
// (device, stream) workspace, growing it when the call needs more of either.
// Growing allocates a new buffer, clears its flagged region with a fill kernel
// (no memset node), and retires the old buffer without freeing it, so it never
// waits for the stream.
int acquire_workspace(int device, hipStream_t stream, int64_t flag_bytes, int64_t data_bytes,
                      uint64_t **flags, float **data) {
    *flags = nullptr;
    *data = nullptr;
    if (flag_bytes == 0 && data_bytes == 0) return ATTN_DECODE_OK;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &ws = g_ws[std::make_pair(device, (void *)stream)];
    const int64_t have_data = (int64_t)ws.bytes - ws.flag_bytes;
    if (ws.ptr == nullptr || ws.flag_bytes < flag_bytes || have_data < data_bytes) {
        int64_t fb = std::max<int64_t>(flag_bytes + flag_bytes / 4, ws.flag_bytes);
        fb = (fb + 0xFFFF) & ~int64_t(0xFFFF);
        int64_t want = std::max<int64_t>(data_bytes + data_bytes / 4, have_data);
        want = (want + 0xFFFF) & ~int64_t(0xFFFF);
        const size_t bytes = (size_t)(fb + want);
        void *p = nullptr;
        hipError_t e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(ATTN_DECODE_ENOMEM, "workspace hipMalloc of " + std::to_string(bytes) + " bytes: " + hipGetErrorString(e));
        }
        if (fb > 0) {
            const int64_t words = fb / 4;
            hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                               static_cast<uint32_t *>(p), words, 0u);
            e = hipGetLastError();
            if (e != hipSuccess) {
                (void)hipFree(p);
                return fail(ATTN_DECODE_EHIP, std::string("flag region fill launch: ") + hipGetErrorString(e));
            }
        }
        if (ws.ptr != nullptr) g_retired.push_back(std::make_pair(device, ws.ptr));
        ws.ptr = p;
        ws.bytes = bytes;
        ws.flag_bytes = fb;
    }
    *flags = static_cast<uint64_t *>(ws.ptr);
    *data = reinterpret_cast<float *>(static_cast<char *>(ws.ptr) + ws.flag_bytes);
    return ATTN_DECODE_OK;
}

// ------------------------------------------------------------ no-allocation scratch

// The partials of attn_decode_noalloc: file-scope device memory of a fixed size,
// one copy on each GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.
constexpr int64_t kNoAllocScratchBytes = ATTN_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
std::map<int, void *> g_scratch_ptr;   // device -> address of its copy of `scratch`

int scratch_on_device(int device, void **ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    auto it = g_scratch_ptr.find(device);
    if (it != g_scratch_ptr.end()) {
        *ptr = it->second;
        return ATTN_DECODE_OK;
    }
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
        return fail(ATTN_DECODE_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[device] = p;
    *ptr = p;
    return ATTN_DECODE_OK;
}

// ------------------------------------------------------------ kernel tables
// Every kernel that reads the query table exists for both table capacities NS.

template <int NS> using partial_fn_t = void (*)(const LaunchArgsT<NS>);
template <int NS> using combine_fn_t = void (*)(const LaunchArgsT<NS>);

template <int D, int VF, int NS>
partial_fn_t<NS> partial_for(int QB, int GB) {
    if (QB == 1) {
        switch (GB) {
            case 1: return attn_partial_kernel<D, 1, 1, VF, NS>;
            case 2: return attn_partial_kernel<D, 1, 2, VF, NS>;
            case 4: return attn_partial_kernel<D, 1, 4, VF, NS>;
        }
    } else if (QB == 2 && GB == 2) {
        return attn_partial_kernel<D, 2, 2, VF, NS>;
    } else if (QB == 4 && GB == 1) {
        return attn_partial_kernel<D, 4, 1, VF, NS>;
    }
    return nullptr;
}

template <int D, int NS>
partial_fn_t<NS> partial_for_format(int vf, int QB, int GB) {
    switch (vf) {
        case kVF16: return partial_for<D, kVF16, NS>(QB, GB);
        case kVI8: return partial_for<D, kVI8, NS>(QB, GB);
        case kVCB: return partial_for<D, kVCB, NS>(QB, GB);
    }
    return nullptr;
}

template <int NS>
partial_fn_t<NS> select_partial(int D, int QB, int GB, int vf) {
    switch (D) {
        case 64: return partial_for_format<64, NS>(vf, QB, GB);
        case 128: return partial_for_format<128, NS>(vf, QB, GB);
        case 256: return partial_for_format<256, NS>(vf, QB, GB);
        case 512: return partial_for_format<512, NS>(vf, QB, GB);
    }
    return nullptr;
}

// The single-buffer lane kernel: head_dim 256, one-byte V, one query per workgroup and one or two
// heads (the launches single_pass_positions admits).
static_assert(kWaves * Geometry<256, kVI8>::RW == 64 && kWaves * Geometry<256, kVCB>::RW == 64,
              "one iteration of one-byte V at head_dim 256 covers the planner's single_pass_positions");
template <int NS>
partial_fn_t<NS> select_partial_single(int D, int GB, int vf) {
    if (D != 256) return nullptr;
    if (vf == kVI8)
        return GB == 1 ? attn_partial_single_kernel<256, 1, kVI8, NS>
                       : GB == 2 ? attn_partial_single_kernel<256, 2, kVI8, NS> : nullptr;
    if (vf == kVCB)
        return GB == 1 ? attn_partial_single_kernel<256, 1, kVCB, NS>
                       : GB == 2 ? attn_partial_single_kernel<256, 2, kVCB, NS> : nullptr;
    return nullptr;
}

template <int D, int NS>
partial_fn_t<NS> mfma_for_format(int vf) {
    switch (vf) {
        case kVF16: return attn_partial_mfma_kernel<D, kVF16, NS>;
        case kVI8: return attn_partial_mfma_kernel<D, kVI8, NS>;
        case kVCB: return attn_partial_mfma_kernel<D, kVCB, NS>;
    }
    return nullptr;
}

template <int NS>
partial_fn_t<NS> select_partial_mfma(int D, int vf) {
    switch (D) {
        case 128: return mfma_for_format<128, NS>(vf);
        case 256: return mfma_for_format<256, NS>(vf);
        case 512: return mfma_for_format<512, NS>(vf);
    }
    return nullptr;
}

template <int NS>
combine_fn_t<NS> select_combine(int D) {
    switch (D) {
        case 64: return attn_combine_kernel<64, NS>;
        case 128: return attn_combine_kernel<128, NS>;
        case 256: return attn_combine_kernel<256, NS>;
        case 512: return attn_combine_kernel<512, NS>;
    }
    return nullptr;
}

// ------------------------------------------------------------ validation helpers

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// How V is stored: fp16 values; int8 codes with fp16 block scales; or
// codebook indices with fp32 block norms and a table of 2^bits levels.
struct VSource {
    const void *v = nullptr;
    int format = kVF16;
    const void *side = nullptr;        // int8: scales; codebook: norms
    const float *codebook = nullptr;
    int32_t bits = 0;

    static VSource plain_or_int8(const void *v, const void *v_scales) {
        VSource s;
        s.v = v;
        s.format = v_scales ? kVI8 : kVF16;
        s.side = v_scales;
        return s;
    }
    uint64_t bytes(uint64_t kv_elems) const { return kv_elems * (format == kVF16 ? 2 : 1); }
    uint64_t side_bytes(uint64_t kv_elems, int32_t D) const {
        if (format == kVI8) return kv_elems / kQuantBlock * 2;
        if (format == kVCB) return kv_elems / (D < 256 ? D : 256) * 4;
        return 0;
    }
};

// Everything after the layout-specific checks: plan, workspace, launches.
// What every launch of one call shares.
struct CallArgs {
    const void *q = nullptr;
    const void *k = nullptr;
    VSource vsrc;
    float *out = nullptr;
    float *ws_o = nullptr;
    float *ws_ml = nullptr;
    uint64_t *flags = nullptr;
    int32_t n_q = 0, n_kv = 0, D = 0;
    float scale_log2 = 0.f;
};

// A launch group of at most kSmallTableSlots query rows takes the small query table.
bool small_table(const LaunchGroup &lg) { return (int)lg.slots.size() <= kSmallTableSlots; }

// The kernels of one table capacity that a plan's launch groups of that capacity use.
template <int NS>
struct Kernels {
    partial_fn_t<NS> mfma = nullptr, lanes = nullptr, single = nullptr;
    combine_fn_t<NS> combine = nullptr;
};

template <int NS>
bool pick_kernels(const CallPlan &plan, int D, int vf, Kernels<NS> &k) {
    const bool small = NS == kSmallTableSlots;
    bool mfma = false, lanes = false, single = false, combine = false;
    for (const LaunchGroup &lg : plan.groups) {
        if (small_table(lg) != small) continue;
        (lg.mfma ? mfma : lanes) = true;
        single = single || lg.single;
        combine = combine || lg.combine_rows > 0;
    }
    if (mfma && (k.mfma = select_partial_mfma<NS>(D, vf)) == nullptr) return false;
    if (lanes && (k.lanes = select_partial<NS>(D, plan.lanes.QB, plan.lanes.GB, vf)) == nullptr) return false;
    if (single && (k.single = select_partial_single<NS>(D, plan.lanes.GB, vf)) == nullptr) return false;
    if (combine && (k.combine = select_combine<NS>(D)) == nullptr) return false;
    return true;
}

// Fills the query table of one launch group and enqueues its partial kernel, or (combine) its
// combine kernel.
template <int NS>
int enqueue_group(const CallPlan &plan, const LaunchGroup &lg, bool combine, const CallArgs &c,
                  const Kernels<NS> &kn, hipStream_t stream) {
    LaunchArgsT<NS> args;
    std::memset(&args, 0, sizeof(args));
    args.q = static_cast<const uint16_t *>(c.q);
    args.k = static_cast<const uint16_t *>(c.k);
    args.v = c.vsrc.v;
    args.vs = c.vsrc.side;
    args.codebook = c.vsrc.codebook;
    args.cb_mask = c.vsrc.format == kVCB ? (1 << c.vsrc.bits) - 1 : 0;
    args.cb_scale = (float)(1.0 / std::sqrt((double)(c.D < 256 ? c.D : 256)));
    args.out = c.out;
    args.ws_o = c.ws_o;
    args.ws_ml = c.ws_ml;
    args.flags = c.flags;
    args.n_q = c.n_q;
    args.G = plan.G;
    args.scale_log2 = c.scale_log2;

    // Search keys: the entries' first work items (partial kernels) or first combine rows
    // (combine kernel); tkey, the first rows among a single-launch grid's merge workgroups.
    const KernelShape &ks = lg.mfma ? plan.matrix : plan.lanes;
    args.n_sub = ks.n_sub;
    args.n_slots = (int32_t)lg.slots.size();
    int32_t item = 0, comb = 0, tail = 0;
    int32_t lead_pos = 0;
    for (size_t i = 0; i < lg.slots.size(); ++i) {
        const int32_t s = lg.slots[i];
        const SlotPlan &sp = plan.slots[s];
        SlotDesc &sd = args.slot[i];
        if (sp.group_n > 0) lead_pos = (int32_t)i;   // a leader or an ungrouped query
        sd.kv_row0 = sp.kv_row0;
        sd.part_row0 = sp.part_row0;
        sd.L = sp.L;
        sd.lo = sp.lo;
        sd.chunk = sp.chunk;
        sd.n_chunks = sp.n_chunks;
        sd.item_begin = sp.group_n > 0 ? item : args.slot[lead_pos].item_begin;
        sd.comb_begin = sp.fused ? tail : comb;
        sd.flag_row0 = sp.fused ? sp.flag_row0 : -1;
        sd.slot_idx = s;
        sd.kv_stride = sp.kv_stride;
        sd.ring_cap = sp.ring_cap;
        sd.ring_base = sp.ring_base;
        sd.group_n = (int16_t)sp.group_n;
        sd.lead_off = (int16_t)(i - lead_pos);
        args.key[i] = combine ? comb : sd.item_begin;
        args.tkey[i] = tail;
        if (sp.group_n > 0) item += c.n_kv * ks.n_sub * sp.n_chunks;
        if (sp.n_chunks > 1) (sp.fused ? tail : comb) += c.n_q;
    }
    args.n_items = item;

    if (combine) {
        hipLaunchKernelGGL(kn.combine, dim3((unsigned)(lg.combine_rows * (c.D / kCombineDims))),
                           dim3(kCombineThreads), 0, stream, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(ATTN_DECODE_EHIP, std::string("combine kernel launch: ") + hipGetErrorString(e));
        return ATTN_DECODE_OK;
    }
    const int64_t grid = lg.items + lg.tail_rows * merge_groups(c.D);   // partial, then merge workgroups
    const int threads = lg.mfma ? kThreads * mfma_dim_splits(c.D) : kThreads;
    hipLaunchKernelGGL(lg.mfma ? kn.mfma : lg.single ? kn.single : kn.lanes, dim3((unsigned)grid), dim3(threads), 0,
                       stream, args);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ATTN_DECODE_EHIP, std::string("partial kernel launch: ") + hipGetErrorString(e));
    return ATTN_DECODE_OK;
}

// no_alloc: the partials go to this device's `scratch` instead of the stream's
// workspace, and the call neither allocates nor frees anything.
int launch(const std::vector<QuerySpan> &spans, const void *q, const void *k_cache,
           const VSource &vsrc, float *out, int32_t n_q, int32_t n_kv,
           int32_t D, float scale, void *stream_ptr, const attn_decode_options *opts,
           bool no_alloc = false) {
    const int32_t chunk = opts ? opts->chunk : 0;
    const int32_t merge_mode = opts ? opts->merge_mode : 0;
    const int32_t path = opts ? opts->path : 0;

    CallPlan plan;
    std::string err = make_plan(spans, n_q, n_kv, D, chunk, merge_mode, plan, path, vsrc.format != kVF16);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    if (no_alloc && plan.workspace_bytes > kNoAllocScratchBytes)
        return fail(ATTN_DECODE_EINVAL, "the call needs " + std::to_string(plan.workspace_bytes) +
                                            " bytes of partials, more than the " +
                                            std::to_string(kNoAllocScratchBytes) +
                                            " bytes of scratch of attn_decode_noalloc");

    Kernels<kSmallTableSlots> small;
    Kernels<kMaxSlotsPerLaunch> large;
    if (!pick_kernels(plan, D, vsrc.format, small) || !pick_kernels(plan, D, vsrc.format, large))
        return fail(ATTN_DECODE_EINVAL, "no kernel for this shape");

    // ---- HIP from here on
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(ATTN_DECODE_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    uint64_t *flags = nullptr;
    float *ws_o = nullptr;
    const int64_t data_bytes = plan.part_rows * (int64_t)(D + 2) * (int64_t)sizeof(float);
    if (no_alloc) {
        void *p = nullptr;
        const int rc = scratch_on_device(device, &p);
        if (rc != ATTN_DECODE_OK) return rc;
        ws_o = static_cast<float *>(p);   // plain partials only: this entry point merges in the combine kernel
    } else {
        const int rc = acquire_workspace(device, stream, flag_region_bytes(plan.flag_rows, D), data_bytes, &flags,
                                         &ws_o);
        if (rc != ATTN_DECODE_OK) return rc;
    }

    CallArgs c;
    c.q = q;
    c.k = k_cache;
    c.vsrc = vsrc;
    c.out = out;
    c.ws_o = ws_o;
    c.ws_ml = ws_o ? ws_o + plan.part_rows * D : nullptr;
    c.flags = flags;
    c.n_q = n_q;
    c.n_kv = n_kv;
    c.D = D;
    c.scale_log2 = (float)((double)scale * 1.4426950408889634074);   // scale * log2(e)

    if (opts && opts->ev_partial_begin) {
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(opts->ev_partial_begin), stream);
        if (e != hipSuccess) return fail(ATTN_DECODE_EHIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
    }
    for (const LaunchGroup &lg : plan.groups) {
        const int rc = small_table(lg) ? enqueue_group(plan, lg, false, c, small, stream)
                                       : enqueue_group(plan, lg, false, c, large, stream);
        if (rc != ATTN_DECODE_OK) return rc;
    }
    if (opts && opts->ev_partial_end) {
        e = hipEventRecord(reinterpret_cast<hipEvent_t>(opts->ev_partial_end), stream);
        if (e != hipSuccess) return fail(ATTN_DECODE_EHIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
    }
    for (const LaunchGroup &lg : plan.groups) {
        if (lg.combine_rows == 0) continue;
        const int rc = small_table(lg) ? enqueue_group(plan, lg, true, c, small, stream)
                                       : enqueue_group(plan, lg, true, c, large, stream);
        if (rc != ATTN_DECODE_OK) return rc;
    }
    return ATTN_DECODE_OK;
}

// Pointer checks shared by both layouts: NULLs, alignment, and out overlapping an input.
int check_pointers(const void *q, const void *k_cache, const VSource &vsrc,
                   const float *out, uint64_t n_rows_q, int32_t n_q, int32_t D, uint64_t kv_elems) {
    const uint64_t q_bytes = n_rows_q * n_q * D * 2;
    const uint64_t out_bytes = n_rows_q * n_q * D * 4;
    const uint64_t k_bytes = kv_elems * 2;
    const uint64_t v_bytes = vsrc.bytes(kv_elems);
    const uint64_t s_bytes = vsrc.side_bytes(kv_elems, D);
    const uint64_t cb_bytes = vsrc.format == kVCB ? (uint64_t(4) << vsrc.bits) : 0;
    if (q == nullptr) return fail(ATTN_DECODE_EINVAL, "q is NULL");
    if (out == nullptr) return fail(ATTN_DECODE_EINVAL, "out is NULL");
    if (kv_elems > 0 && (k_cache == nullptr || vsrc.v == nullptr))
        return fail(ATTN_DECODE_EINVAL, "k_cache / v_cache is NULL");
    if (!aligned(q, 16) || !aligned(out, 16)) return fail(ATTN_DECODE_EINVAL, "q and out must be 16-byte aligned");
    if (!aligned(k_cache, 16) || !aligned(vsrc.v, 16))
        return fail(ATTN_DECODE_EINVAL, "k_cache and v_cache must be 16-byte aligned");
    if (vsrc.format == kVI8 && !aligned(vsrc.side, 2))
        return fail(ATTN_DECODE_EINVAL, "v_scales must be 2-byte aligned");
    if (vsrc.format == kVCB) {
        if (kv_elems > 0 && vsrc.side == nullptr) return fail(ATTN_DECODE_EINVAL, "v_norms is NULL");
        if (vsrc.codebook == nullptr) return fail(ATTN_DECODE_EINVAL, "codebook is NULL");
        if (!aligned(vsrc.side, 4) || !aligned(vsrc.codebook, 4))
            return fail(ATTN_DECODE_EINVAL, "v_norms and codebook must be 4-byte aligned");
    }
    if (overlaps(out, out_bytes, q, q_bytes) || overlaps(out, out_bytes, k_cache, k_bytes) ||
        overlaps(out, out_bytes, vsrc.v, v_bytes) || overlaps(out, out_bytes, vsrc.side, s_bytes) ||
        overlaps(out, out_bytes, vsrc.codebook, cb_bytes))
        return fail(ATTN_DECODE_EINVAL, "out overlaps an input");
    return ATTN_DECODE_OK;
}

int run(const void *q, const void *k_cache, const VSource &vsrc,
        const int32_t *seq_lens, int32_t window, float *out, int32_t n_slots, int32_t n_q,
        int32_t n_kv, int32_t D, float scale, void *stream_ptr, const attn_decode_options *opts,
        bool no_alloc = false) {
    g_last_error.clear();
    const int32_t chunk = opts ? opts->chunk : 0;
    const int32_t merge_mode = opts ? opts->merge_mode : 0;

    if (vsrc.format == kVCB && (vsrc.bits < 1 || vsrc.bits > 8))
        return fail(ATTN_DECODE_EINVAL, "codebook_bits must be in 1..8");
    std::string err = check_shapes(seq_lens, n_slots, window, n_q, n_kv, D, vsrc.format == kVI8, chunk,
                                   merge_mode);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    if (!std::isfinite(scale)) return fail(ATTN_DECODE_EINVAL, "scale must be finite");
    if (n_slots == 0) return ATTN_DECODE_OK;

    // sizes (64-bit, overflow-checked)
    uint64_t total_pos = 0;
    for (int32_t s = 0; s < n_slots; ++s) total_pos += (uint64_t)seq_lens[s];
    const uint64_t kv_elems = total_pos * (uint64_t)n_kv * (uint64_t)D;
    if (total_pos > (uint64_t(1) << 40) || kv_elems > (uint64_t(1) << 46))
        return fail(ATTN_DECODE_EINVAL, "KV cache too large");
    int rc = check_pointers(q, k_cache, vsrc, out, (uint64_t)n_slots, n_q, D, kv_elems);
    if (rc != ATTN_DECODE_OK) return rc;

    std::vector<QuerySpan> spans;
    spans_packed(seq_lens, n_slots, window, n_kv, spans);
    return launch(spans, q, k_cache, vsrc, out, n_q, n_kv, D, scale, stream_ptr, opts, no_alloc);
}

int run_cache(const void *q, const void *k_cache, const VSource &vsrc,
              const int32_t *slot_ids, const int32_t *positions, int32_t n_queries,
              int32_t n_cache_slots, int32_t capacity, int32_t ring, int32_t window, float *out,
              int32_t n_q, int32_t n_kv, int32_t D, float scale, void *stream_ptr,
              const attn_decode_options *opts) {
    g_last_error.clear();
    const int32_t chunk = opts ? opts->chunk : 0;
    const int32_t merge_mode = opts ? opts->merge_mode : 0;

    if (vsrc.format == kVCB && (vsrc.bits < 1 || vsrc.bits > 8))
        return fail(ATTN_DECODE_EINVAL, "codebook_bits must be in 1..8");
    if (n_cache_slots < 0) return fail(ATTN_DECODE_EINVAL, "n_cache_slots must be >= 0");
    std::string err = check_common(n_q, n_kv, D, vsrc.format == kVI8, window, chunk, merge_mode);
    if (err.empty()) err = check_cache(slot_ids, positions, n_queries, n_cache_slots, capacity, ring);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    if (!std::isfinite(scale)) return fail(ATTN_DECODE_EINVAL, "scale must be finite");
    if (n_queries == 0) return ATTN_DECODE_OK;

    const uint64_t rows = (uint64_t)n_cache_slots * (uint64_t)n_kv * (uint64_t)capacity;
    const uint64_t kv_elems = rows * (uint64_t)D;
    if (rows > (uint64_t(1) << 40) || kv_elems > (uint64_t(1) << 46))
        return fail(ATTN_DECODE_EINVAL, "KV cache too large");
    int rc = check_pointers(q, k_cache, vsrc, out, (uint64_t)n_queries, n_q, D, kv_elems);
    if (rc != ATTN_DECODE_OK) return rc;

    std::vector<QuerySpan> spans;
    spans_cache(slot_ids, positions, n_queries, capacity, ring, window, n_kv, spans);
    return launch(spans, q, k_cache, vsrc, out, n_q, n_kv, D, scale, stream_ptr, opts);
}

typedef void (*append_fn)(const AppendArgs);

template <int D>
append_fn append_for(int vf) {
    switch (vf) {
        case kVF16: return kv_append_kernel<D, kVF16>;
        case kVI8: return kv_append_kernel<D, kVI8>;
        case kVCB: return kv_append_kernel<D, kVCB>;
    }
    return nullptr;
}

append_fn select_append(int D, int vf) {
    switch (D) {
        case 64: return append_for<64>(vf);
        case 128: return append_for<128>(vf);
        case 256: return append_for<256>(vf);
        case 512: return append_for<512>(vf);
    }
    return nullptr;
}

// Where an append writes V: fp16 values; int8 codes plus fp16 block scales; or
// codebook indices plus fp32 block norms, encoded with `signs` and `codebook`.
struct AppendV {
    void *v = nullptr;
    int format = kVF16;
    void *side = nullptr;              // int8: scales; codebook: norms
    const float *signs = nullptr;
    const float *codebook = nullptr;
    int32_t bits = 0;
};

int run_append(const float *k_new, const float *v_new, void *k_cache, const AppendV &vd,
               const int32_t *slot_ids, const int32_t *positions, int32_t n_rows,
               int32_t n_cache_slots, int32_t capacity, int32_t ring, int32_t n_kv, int32_t D,
               void *stream_ptr) {
    g_last_error.clear();
    if (n_rows < 0) return fail(ATTN_DECODE_EINVAL, "n_rows must be >= 0");
    if (n_cache_slots < 0) return fail(ATTN_DECODE_EINVAL, "n_cache_slots must be >= 0");
    if (n_kv <= 0) return fail(ATTN_DECODE_EINVAL, "n_kv_heads must be positive");
    if (!supported_head_dim(D)) return fail(ATTN_DECODE_EINVAL, "head_dim must be 64, 128, 256 or 512");
    if (vd.format == kVCB && (vd.bits < 1 || vd.bits > 8))
        return fail(ATTN_DECODE_EINVAL, "codebook_bits must be in 1..8");
    std::string err = check_cache(slot_ids, positions, n_rows, n_cache_slots, capacity, ring);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    if (n_rows == 0) return ATTN_DECODE_OK;

    // every new row must land on its own cache row: rows in increasing (slot, cache row) order
    // (a prompt, or one token for each of several slots) pass in one pass; any other order is sorted
    auto dst_of = [&](int32_t i) {
        return std::make_pair(slot_ids[i], ring ? positions[i] % capacity : positions[i]);
    };
    bool increasing = true;
    if (ring) {
        for (int32_t i = 1; i < n_rows && increasing; ++i) increasing = dst_of(i - 1) < dst_of(i);
    } else {   // linear storage: the row is the position
        for (int32_t i = 1; i < n_rows; ++i)
            increasing &= slot_ids[i - 1] < slot_ids[i] || (slot_ids[i - 1] == slot_ids[i] && positions[i - 1] < positions[i]);
    }
    if (!increasing) {
        std::vector<std::pair<int32_t, int32_t>> dst(n_rows);
        for (int32_t i = 0; i < n_rows; ++i) dst[i] = dst_of(i);
        std::sort(dst.begin(), dst.end());
        for (int32_t i = 1; i < n_rows; ++i)
            if (dst[i] == dst[i - 1]) return fail(ATTN_DECODE_EINVAL, "two new rows land on the same cache row");
    }

    const uint64_t rows = (uint64_t)n_cache_slots * (uint64_t)n_kv * (uint64_t)capacity;
    const uint64_t kv_elems = rows * (uint64_t)D;
    if (rows > (uint64_t(1) << 40) || kv_elems > (uint64_t(1) << 46))
        return fail(ATTN_DECODE_EINVAL, "KV cache too large");
    const uint64_t new_bytes = (uint64_t)n_rows * n_kv * D * 4;
    const uint64_t k_bytes = kv_elems * 2, v_bytes = kv_elems * (vd.format == kVF16 ? 2 : 1);
    const uint64_t s_bytes = vd.format == kVI8 ? kv_elems / kQuantBlock * 2
                           : vd.format == kVCB ? kv_elems / (D < 256 ? D : 256) * 4 : 0;
    if (k_new == nullptr || v_new == nullptr) return fail(ATTN_DECODE_EINVAL, "k_new / v_new is NULL");
    if (k_cache == nullptr || vd.v == nullptr) return fail(ATTN_DECODE_EINVAL, "k_cache / v_cache is NULL");
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(ATTN_DECODE_EINVAL, "k_new and v_new must be 16-byte aligned");
    if (!aligned(k_cache, 16) || !aligned(vd.v, 16))
        return fail(ATTN_DECODE_EINVAL, "k_cache and v_cache must be 16-byte aligned");
    if (vd.format == kVI8 && !aligned(vd.side, 2)) return fail(ATTN_DECODE_EINVAL, "v_scales must be 2-byte aligned");
    const uint64_t cb_bytes = vd.format == kVCB ? (uint64_t(4) << vd.bits) : 0;
    const uint64_t sg_bytes = vd.format == kVCB ? (uint64_t)D * 4 : 0;
    if (vd.format == kVCB) {
        if (vd.side == nullptr || vd.signs == nullptr || vd.codebook == nullptr)
            return fail(ATTN_DECODE_EINVAL, "v_norms / signs / codebook is NULL");
        if (!aligned(vd.side, 4) || !aligned(vd.signs, 4) || !aligned(vd.codebook, 4))
            return fail(ATTN_DECODE_EINVAL, "v_norms, signs and codebook must be 4-byte aligned");
    }
    // inputs (new rows, and for codebook V the signs and levels) against the three outputs
    const void *ins[4] = {k_new, v_new, vd.signs, vd.codebook};
    const uint64_t in_bytes[4] = {new_bytes, new_bytes, sg_bytes, cb_bytes};
    const void *outs[3] = {k_cache, vd.v, vd.side};
    const uint64_t out_bytes[3] = {k_bytes, v_bytes, s_bytes};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 4; ++b)
            if (overlaps(ins[b], in_bytes[b], outs[a], out_bytes[a]))
                return fail(ATTN_DECODE_EINVAL, b < 2 ? "k_new / v_new overlaps the cache"
                                                      : "signs / codebook overlaps the cache");
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b]))
                return fail(ATTN_DECODE_EINVAL, "cache arrays overlap");
    }
    const append_fn fn = select_append(D, vd.format);
    if (fn == nullptr) return fail(ATTN_DECODE_EINVAL, "no kernel for this shape");

    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    AppendArgs args;
    std::memset(&args, 0, sizeof(args));
    args.k_new = k_new;
    args.v_new = v_new;
    args.k_cache = static_cast<uint16_t *>(k_cache);
    args.v_cache = vd.v;
    if (vd.format == kVI8) args.v_scales = static_cast<uint16_t *>(vd.side);
    if (vd.format == kVCB) args.v_norms = static_cast<float *>(vd.side);
    args.signs = vd.signs;
    args.codebook = vd.codebook;
    args.cb_bits = vd.bits;
    args.inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
    args.n_kv = n_kv;
    args.capacity = capacity;
    // Rows go out as runs (consecutive cache rows of one slot), up to kAppendMaxRuns runs and
    // kAppendMaxLaunchRows rows per launch.
    constexpr int32_t kAppendMaxLaunchRows = 1 << 20;
    auto cache_row = [&](int32_t i) {
        const int32_t p = positions[i];
        return (int64_t)slot_ids[i] * n_kv * capacity + (ring ? p % capacity : p);
    };
    int32_t r0 = 0;
    while (r0 < n_rows) {
        args.row0 = r0;
        int32_t nr = 0, runs = 0;
        int64_t next = -1;   // cache row that would continue the current run
        while (r0 + nr < n_rows && nr < kAppendMaxLaunchRows) {
            const int64_t cr = cache_row(r0 + nr);
            const bool same_run = runs > 0 && cr == next && slot_ids[r0 + nr] == slot_ids[r0 + nr - 1];
            if (!same_run) {
                if (runs == kAppendMaxRuns) break;
                args.run[runs].cache_row0 = cr;
                args.run[runs].row_begin = nr;
                ++runs;
            }
            next = cr + 1;
            ++nr;
        }
        args.n_rows = nr;
        args.n_runs = runs;
        const int64_t units = (int64_t)nr * n_kv;
        hipLaunchKernelGGL(fn, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, args);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(ATTN_DECODE_EHIP, std::string("append kernel launch: ") + hipGetErrorString(e));
        r0 += nr;
    }
    return ATTN_DECODE_OK;
}

}  // namespace

// ============================================================ C ABI

extern "C" int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                           const void *v_scales, const int32_t *seq_lens, int32_t window,
                           float *out, int32_t n_slots, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, float scale, void *stream) {
    return run(q, k_cache, VSource::plain_or_int8(v_cache, v_scales), seq_lens, window, out, n_slots, n_q_heads,
               n_kv_heads, head_dim, scale, stream, nullptr);
}

extern "C" int attn_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                              const void *v_scales, const int32_t *seq_lens, int32_t window,
                              float *out, int32_t n_slots, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, float scale, void *stream,
                              const attn_decode_options *opts) {
    return run(q, k_cache, VSource::plain_or_int8(v_cache, v_scales), seq_lens, window, out, n_slots, n_q_heads,
               n_kv_heads, head_dim, scale, stream, opts);
}

extern "C" int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                   const void *v_scales, const int32_t *seq_lens, int32_t window,
                                   float *out, int32_t n_slots, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, float scale, void *stream,
                                   const attn_decode_options *opts) {
    if (opts && opts->merge_mode == kMergeInKernel) {
        g_last_error.clear();
        return fail(ATTN_DECODE_EINVAL, "attn_decode_noalloc merges in the combine kernel: merge_mode must be 0 or 1");
    }
    return run(q, k_cache, VSource::plain_or_int8(v_cache, v_scales), seq_lens, window, out, n_slots, n_q_heads,
               n_kv_heads, head_dim, scale, stream, opts, true);
}

extern "C" int attn_decode_cb(const void *q, const void *k_cache, const void *v_codes,
                              const float *v_norms, const float *codebook, int32_t codebook_bits,
                              const int32_t *seq_lens, int32_t window, float *out, int32_t n_slots,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                              void *stream, const attn_decode_options *opts) {
    VSource vsrc;
    vsrc.v = v_codes;
    vsrc.format = kVCB;
    vsrc.side = v_norms;
    vsrc.codebook = codebook;
    vsrc.bits = codebook_bits;
    return run(q, k_cache, vsrc, seq_lens, window, out, n_slots, n_q_heads, n_kv_heads, head_dim,
               scale, stream, opts);
}

extern "C" int attn_fwht_undo(const float *x, const float *signs, float *y, int64_t n_rows,
                              int32_t head_dim, void *stream) {
    g_last_error.clear();
    typedef void (*undo_fn)(const float *, const float *, float *, int64_t, float);
    undo_fn fn = nullptr;
    switch (head_dim) {
        case 64: fn = fwht_undo_kernel<64>; break;
        case 128: fn = fwht_undo_kernel<128>; break;
        case 256: fn = fwht_undo_kernel<256>; break;
        case 512: fn = fwht_undo_kernel<512>; break;
        default: return fail(ATTN_DECODE_EINVAL, "head_dim must be 64, 128, 256 or 512");
    }
    if (n_rows < 0) return fail(ATTN_DECODE_EINVAL, "n_rows must be >= 0");
    if (n_rows > (int64_t)4 * 0x7fffffff) return fail(ATTN_DECODE_EINVAL, "n_rows too large");
    if (n_rows == 0) return ATTN_DECODE_OK;
    if (x == nullptr || signs == nullptr || y == nullptr) return fail(ATTN_DECODE_EINVAL, "x / signs / y is NULL");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(ATTN_DECODE_EINVAL, "x and y must be 16-byte aligned");
    if (!aligned(signs, 4)) return fail(ATTN_DECODE_EINVAL, "signs must be 4-byte aligned");
    const uint64_t bytes = (uint64_t)n_rows * (uint64_t)head_dim * 4;
    if (x != y && overlaps(x, bytes, y, bytes)) return fail(ATTN_DECODE_EINVAL, "y overlaps x without being x");
    if (overlaps(y, bytes, signs, (uint64_t)head_dim * 4)) return fail(ATTN_DECODE_EINVAL, "y overlaps signs");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const float inv = (float)(1.0 / std::sqrt((double)head_dim));
    hipLaunchKernelGGL(fn, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, st, x, signs, y, n_rows, inv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ATTN_DECODE_EHIP, std::string("fwht undo launch: ") + hipGetErrorString(e));
    return ATTN_DECODE_OK;
}

extern "C" int attn_decode_cache(const void *q, const void *k_cache, const void *v_cache,
                                 const void *v_scales, const int32_t *slot_ids,
                                 const int32_t *positions, int32_t n_queries, int32_t n_cache_slots,
                                 int32_t capacity, int32_t ring, int32_t window, float *out,
                                 int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                                 void *stream, const attn_decode_options *opts) {
    return run_cache(q, k_cache, VSource::plain_or_int8(v_cache, v_scales), slot_ids, positions, n_queries,
                     n_cache_slots, capacity, ring, window, out, n_q_heads, n_kv_heads, head_dim, scale, stream,
                     opts);
}

extern "C" int attn_decode_cache_cb(const void *q, const void *k_cache, const void *v_codes,
                                    const float *v_norms, const float *codebook, int32_t codebook_bits,
                                    const int32_t *slot_ids, const int32_t *positions, int32_t n_queries,
                                    int32_t n_cache_slots, int32_t capacity, int32_t ring, int32_t window,
                                    float *out, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    float scale, void *stream, const attn_decode_options *opts) {
    VSource vsrc;
    vsrc.v = v_codes;
    vsrc.format = kVCB;
    vsrc.side = v_norms;
    vsrc.codebook = codebook;
    vsrc.bits = codebook_bits;
    return run_cache(q, k_cache, vsrc, slot_ids, positions, n_queries, n_cache_slots, capacity, ring, window,
                     out, n_q_heads, n_kv_heads, head_dim, scale, stream, opts);
}

extern "C" int attn_kv_append(const float *k_new, const float *v_new, void *k_cache, void *v_cache,
                              void *v_scales, const int32_t *slot_ids, const int32_t *positions,
                              int32_t n_rows, int32_t n_cache_slots, int32_t capacity, int32_t ring,
                              int32_t n_kv_heads, int32_t head_dim, void *stream) {
    AppendV vd;
    vd.v = v_cache;
    vd.format = v_scales ? kVI8 : kVF16;
    vd.side = v_scales;
    return run_append(k_new, v_new, k_cache, vd, slot_ids, positions, n_rows, n_cache_slots, capacity, ring,
                      n_kv_heads, head_dim, stream);
}

extern "C" int attn_kv_append_cb(const float *k_new, const float *v_new, void *k_cache, void *v_codes,
                                 float *v_norms, const float *signs, const float *codebook,
                                 int32_t codebook_bits, const int32_t *slot_ids, const int32_t *positions,
                                 int32_t n_rows, int32_t n_cache_slots, int32_t capacity, int32_t ring,
                                 int32_t n_kv_heads, int32_t head_dim, void *stream) {
    AppendV vd;
    vd.v = v_codes;
    vd.format = kVCB;
    vd.side = v_norms;
    vd.signs = signs;
    vd.codebook = codebook;
    vd.bits = codebook_bits;
    return run_append(k_new, v_new, k_cache, vd, slot_ids, positions, n_rows, n_cache_slots, capacity, ring,
                      n_kv_heads, head_dim, stream);
}

extern "C" int attn_decode_plan(const int32_t *seq_lens, int32_t n_slots, int32_t window,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                int32_t v_int8, int32_t chunk, int32_t *chunk_keys,
                                int32_t *n_chunks, int64_t *workspace_bytes,
                                int64_t *n_partial_workgroups) {
    g_last_error.clear();
    std::string err = check_shapes(seq_lens, n_slots, window, n_q_heads, n_kv_heads, head_dim,
                                   v_int8 != 0, chunk);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    CallPlan plan;
    std::vector<QuerySpan> spans;
    spans_packed(seq_lens, n_slots, window, n_kv_heads, spans);
    err = make_plan(spans, n_q_heads, n_kv_heads, head_dim, chunk, kMergeAuto, plan, kPathAuto, v_int8 != 0);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    for (int32_t s = 0; s < n_slots; ++s) {
        if (chunk_keys) chunk_keys[s] = plan.slots[s].chunk;
        if (n_chunks) n_chunks[s] = plan.slots[s].n_chunks;
    }
    if (workspace_bytes) *workspace_bytes = plan.workspace_bytes;
    if (n_partial_workgroups) *n_partial_workgroups = plan.total_items;
    return ATTN_DECODE_OK;
}

extern "C" int attn_decode_cache_plan(const int32_t *slot_ids, const int32_t *positions, int32_t n_queries,
                                      int32_t n_cache_slots, int32_t capacity, int32_t ring, int32_t window,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t v_format,
                                      int32_t chunk, int32_t *chunk_keys, int32_t *n_chunks, int32_t *kernel,
                                      int32_t *group_leader, int64_t *workspace_bytes,
                                      int64_t *n_partial_workgroups) {
    g_last_error.clear();
    if (v_format < kVF16 || v_format > kVCB)
        return fail(ATTN_DECODE_EINVAL, "v_format must be 0 (fp16), 1 (int8) or 2 (codebook)");
    if (n_cache_slots < 0) return fail(ATTN_DECODE_EINVAL, "n_cache_slots must be >= 0");
    std::string err = check_common(n_q_heads, n_kv_heads, head_dim, v_format == kVI8, window, chunk, 0);
    if (err.empty()) err = check_cache(slot_ids, positions, n_queries, n_cache_slots, capacity, ring);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    CallPlan plan;
    std::vector<QuerySpan> spans;
    spans_cache(slot_ids, positions, n_queries, capacity, ring, window, n_kv_heads, spans);
    err = make_plan(spans, n_q_heads, n_kv_heads, head_dim, chunk, kMergeAuto, plan, kPathAuto, v_format != kVF16);
    if (!err.empty()) return fail(ATTN_DECODE_EINVAL, err);
    for (int32_t i = 0; i < n_queries; ++i) {
        const SlotPlan &sp = plan.slots[i];
        if (chunk_keys) chunk_keys[i] = sp.chunk;
        if (n_chunks) n_chunks[i] = sp.n_chunks;
        if (kernel) kernel[i] = sp.mfma ? 1 : 0;
        if (group_leader) group_leader[i] = sp.group_n > 0 ? i : sp.leader;
    }
    if (workspace_bytes) *workspace_bytes = plan.workspace_bytes;
    if (n_partial_workgroups) *n_partial_workgroups = plan.total_items;
    return ATTN_DECODE_OK;
}

extern "C" const char *attn_decode_last_error(void) { return g_last_error.c_str(); }

extern "C" int attn_decode_release(void) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int rc = ATTN_DECODE_OK;
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    std::vector<std::pair<int, void *>> bufs = g_retired;
    for (auto &kv : g_ws)
        if (kv.second.ptr != nullptr) bufs.push_back(std::make_pair(kv.first.first, kv.second.ptr));
    std::sort(bufs.begin(), bufs.end());
    int synced = -1;
    for (const auto &b : bufs) {
        hipError_t e = hipSuccess;
        if (b.first != synced) {   // every device that owns a buffer, once
            e = hipSetDevice(b.first);
            if (e == hipSuccess) e = hipDeviceSynchronize();
            synced = b.first;
        }
        if (e == hipSuccess) e = hipFree(b.second);
        if (e != hipSuccess) rc = fail(ATTN_DECODE_EHIP, std::string("release: ") + hipGetErrorString(e));
    }
    g_ws.clear();
    g_retired.clear();
    if (have_cur) (void)hipSetDevice(cur);
    return rc;
}
