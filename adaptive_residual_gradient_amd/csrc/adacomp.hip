// C ABI of the AdaComp library (declared in include/adacomp.h): plan
// management, argument checking and stream-ordered kernel launches.
//
// Method: "AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
// page, definition paragraph and Mechanism claim on local-bin soft threshold
// and mean-g_max quantization (Algorithm 2); index word widths from its
// Application claim (Table 2).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/adacomp.h"
#include "kernels.hpp"
#include "layout.hpp"

using adacomp::Layout;
using adacomp::SegDev;

// Device copies of one tiling's tables.
struct DevTiling {
    uint32_t* tile_seg = nullptr;
    uint32_t* vtiles[adacomp::kVariants] = {nullptr, nullptr, nullptr};
    uint32_t* chunk_tile_begin = nullptr;
    uint32_t* chunk_seg = nullptr;
};

struct adacomp_plan {
    Layout L;
    int device = -1;
    void* dmem = nullptr;
    SegDev* d_segs = nullptr;
    adacomp::CountChunk* d_cchunks = nullptr;   // decode count chunks
    DevTiling dct, ddt;                                        // compress and decode tiles
    adacomp::DecDesc* ddesc[adacomp::kDecVariants] = {nullptr, nullptr};   // decode tiles in launch order
    uint32_t tile_lds_words[adacomp::kVariants] = {0, 0, 0};  // one tile's LDS words
    adacomp::Finish finish = adacomp::Finish::kSeparate;
    uint32_t* tile_t0 = nullptr;    // small-table finish: first element of each compress tile
    uint32_t small_lds_bytes = 0;   // k_finish_small's dynamic LDS
    uint32_t single_lds_bytes = 0;  // k_compress_single's: tile or finish tables, the larger
    uint32_t chunk_lds_bytes = 0;   // k_finish_chunks' dynamic LDS
    // Plain sums of up to 16 messages take k_decode_tiles_sum: plans with at least
    // kSumKernelMinTiles LDS decode tiles, all of 16-bit words, or made with
    // ADACOMP_PLAN_DECODE_RECORDS.  Measured on MI355X
    // (K = 16, step-10 messages): 1.07e9 elements at L_T 500, 1.30 -> 1.15 ms; at L_T 50
    // (8-bit words, dense tiles) 2.12 -> 2.32 ms; 25e6 elements at L_T 500, 51.6 -> 57.6 us.
    bool sum_kernel = false;
    // k_decode_count requests a decode tile's count blocks together on tables of at least
    // kSumKernelMinTiles decode tiles where some tile's count words span more than
    // kCountBatchMinBytes (dense short bins).  Measured on MI355X (K = 16, step-10 messages):
    // 1.07e9 elements at L_T 50, decode 2.114 -> 2.055 ms; the conv-stack and ResNet-50 tables
    // (fewer tiles) 36.3 -> 38.0 us and 107.3 -> 109.1 us, so they keep one block at a time.
    bool count_batched = false;
    // Some layer's decode tiles (LDS tiles) hold 8-bit entry words: k_decode_tiles then
    // reserves its per-entry bin table.
    bool dense_words = false;
};
constexpr uint32_t kCountBatchMinBytes = 48;
constexpr uint64_t kSumKernelMinTiles = 65536;

namespace adacomp {
// NTS: non-temporal residue stores (tables past kCachedResidueMaxElems).
template <int V, bool NTS>
hipError_t launch_tile_pass_nts(const adacomp_plan* plan, hipStream_t stream, float* residue,
                                const float* dW, uint8_t* msg, uint32_t* stage, uint32_t* tile_cnt,
                                double* tile_gsum, float* bin_max_out) {
    const uint32_t n = static_cast<uint32_t>(plan->L.ct.by_variant[V].size());
    constexpr uint32_t CV = kVarThreads[2] * kVarVecs[2];   // float4 per chunk of shape 2
    if (V == 2 && plan->L.ct.max_span_vecs[2] <= kLongRegChunks * CV)
        // long bins of at most kLongRegChunks chunks: one bin per workgroup, held in registers
        hipLaunchKernelGGL((k_tile_pass_long<kVarThreads[2], kVarVecs[2], kLongRegChunks, NTS>),
                           dim3(n), dim3(kVarThreads[2]), 0, stream, plan->d_segs,
                           plan->dct.tile_seg, plan->dct.vtiles[2], residue, dW, msg, stage,
                           tile_cnt, tile_gsum, bin_max_out);
    else if (V == 2 && plan->L.ct.max_span_vecs[2] <= kLongRegChunks * 4 * CV)
        // up to 4 chunks of 1024 x 2 float4 (every L_T up to 32768): 1024-thread workgroups
        hipLaunchKernelGGL((k_tile_pass_long<1024, kVarVecs[2], kLongRegChunks, NTS>), dim3(n),
                           dim3(1024), 0, stream, plan->d_segs, plan->dct.tile_seg,
                           plan->dct.vtiles[2], residue, dW, msg, stage, tile_cnt, tile_gsum,
                           bin_max_out);
    else if (V == 2)   // longer bins: one bin per workgroup, streamed twice in chunks
        hipLaunchKernelGGL((k_tile_pass_long<kVarThreads[2], kVarVecs[2], 0, NTS>), dim3(n),
                           dim3(kVarThreads[2]), 0, stream, plan->d_segs, plan->dct.tile_seg,
                           plan->dct.vtiles[2], residue, dW, msg, stage, tile_cnt, tile_gsum,
                           bin_max_out);
    else
        hipLaunchKernelGGL((k_tile_pass<kVarThreads[V], kVarVecs[V], NTS>), dim3(n),
                           dim3(kVarThreads[V]), plan->tile_lds_words[V] * 4, stream,
                           plan->d_segs, plan->dct.tile_seg, plan->dct.vtiles[V], residue, dW,
                           msg, stage, tile_cnt, tile_gsum, bin_max_out);
    return hipGetLastError();
}

template <int V>
hipError_t launch_tile_pass(const adacomp_plan* plan, hipStream_t stream, float* residue,
                            const float* dW, uint8_t* msg, uint32_t* stage, uint32_t* tile_cnt,
                            double* tile_gsum, float* bin_max_out) {
    if (plan->L.total_numel > kCachedResidueMaxElems)
        return launch_tile_pass_nts<V, true>(plan, stream, residue, dW, msg, stage, tile_cnt,
                                             tile_gsum, bin_max_out);
    return launch_tile_pass_nts<V, false>(plan, stream, residue, dW, msg, stage, tile_cnt,
                                          tile_gsum, bin_max_out);
}
}  // namespace adacomp

// Per-call device timing: one event at the start of a call and one after each
// stage, so consecutive stages share their boundary event.
struct adacomp_timer {
    struct Call {
        std::vector<hipEvent_t> ev;   // ev[0] call start, ev[i + 1] end of stage[i]
        std::vector<int> stage;
        int whole;                    // the whole-call stage, ev.front() .. ev.back()
    };
    std::vector<Call> calls;
    double ms[ADACOMP_NUM_STAGES] = {};
    uint64_t n[ADACOMP_NUM_STAGES] = {};
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range_of(const void* p, uint64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

int check_device(const adacomp_plan* plan) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ADACOMP_ERR_HIP;
    return dev == plan->device ? ADACOMP_OK : ADACOMP_ERR_INVALID_ARGUMENT;
}

// Records the boundary events of one call's stages on its stream.  Any
// event failure switches timing off for the call; launches are unaffected.
struct CallTimer {
    adacomp_timer* t;
    hipStream_t s;
    adacomp_timer::Call c;
    CallTimer(adacomp_timer* timer, hipStream_t stream, int whole) : t(timer), s(stream) {
        c.whole = whole;
        if (t) record();
    }
    void record() {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) {
            drop();
            return;
        }
        c.ev.push_back(e);
        if (hipEventRecord(e, s) != hipSuccess) drop();
    }
    void mark(int stage) {   // end of `stage`, start of the next one
        if (!t) return;
        c.stage.push_back(stage);
        record();
    }
    void finish() {
        if (!t) return;
        if (c.stage.empty()) record();   // a call without stages: its end event
        if (!t) return;                  // that event failed
        t->calls.push_back(std::move(c));
        c = adacomp_timer::Call{};
        t = nullptr;
    }
    void drop() {
        for (hipEvent_t e : c.ev) (void)hipEventDestroy(e);
        c.ev.clear();
        c.stage.clear();
        t = nullptr;
    }
    ~CallTimer() { drop(); }   // a launch failed before finish()
};

// Encode workgroups (4 wavefronts each): about one wavefront per 2048
// elements, at most kEncMaxBlocks.  The survivors are shared out evenly
// among them on the device.
uint32_t encode_blocks(const Layout& L) {
    const uint64_t b = (L.total_numel + 8191) / 8192;
    return static_cast<uint32_t>(std::min<uint64_t>(std::max<uint64_t>(b, 1), adacomp::kEncMaxBlocks));
}

int launch_status() {
    return hipGetLastError() == hipSuccess ? ADACOMP_OK : ADACOMP_ERR_HIP;
}

// Plain decode of long-bin tiles with the whole tile in LDS (one 1024-thread
// workgroup per CU) rather than in place in out: when every long layer puts
// at least two bins in a tile (L_T up to 18432; with one bin per tile a
// single wavefront gathers it and the in-place kernel is faster: L_T =
// 32768, K = 16, 2.87 against 2.39 ms on 1.07e9 elements, while L_T = 5000
// takes 1.50 against 2.60 ms) and the tile's tables fit the 160 KB a
// workgroup may hold (the kernel is allowed that much; if that fails, the
// in-place kernel is used).
bool long_decode_in_lds(const Layout& L, uint32_t K, uint32_t KG, uint32_t ps, int opt) {
    constexpr uint32_t kLdsMax = 160u * 1024u;
    for (const SegDev& sg : L.segs)
        if (sg.dt.variant == 1u && sg.dt.bpt < 2u) return false;
    const uint32_t lds = adacomp::decode_lds_bytes(L.dt.max_span_vecs[1] * 4, K, KG, ps, 16);
    if (lds > kLdsMax) return false;
    const void* fn = opt == adacomp::kOptSgd
                         ? reinterpret_cast<const void*>(&adacomp::k_decode_apply<1024, true, adacomp::kOptSgd>)
                     : opt == adacomp::kOptAdam
                         ? reinterpret_cast<const void*>(&adacomp::k_decode_apply<1024, true, adacomp::kOptAdam>)
                         : reinterpret_cast<const void*>(&adacomp::k_decode_apply<1024, true>);
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsMax)) ==
           hipSuccess;
}

struct DecodeLayout {
    uint64_t status, dcnt, doff, dchunk_cnt, dchunk_base, dseg_s, dseg_eoff, dvalid, drec, total;
};

DecodeLayout decode_layout(const Layout& L, uint32_t K) {
    DecodeLayout d{};
    uint64_t w = 0;
    auto take = [&w](uint64_t bytes) {
        const uint64_t at = w;
        w = adacomp::round_up(w + bytes, adacomp::kAlign);
        return at;
    };
    const uint64_t T = L.dt.ntiles, C = L.dt.nchunks, S = L.nseg;
    d.status = take(4);
    d.dcnt = take(4 * K * T);
    d.doff = take(4 * K * T);
    d.dchunk_cnt = take(4 * K * C);
    d.dchunk_base = take(4 * K * C);
    d.dseg_s = take(4 * K * S);
    d.dseg_eoff = take(8 * K * S);
    d.dvalid = take(4 * uint64_t(K));
    d.drec = take(8 * K * uint64_t(L.dt.by_variant[0].size()));
    d.total = w;
    return d;
}

}  // namespace

extern "C" {

const char* adacomp_status_str(int status) {
    switch (status) {
        case ADACOMP_OK: return "ok";
        case ADACOMP_ERR_INVALID_ARGUMENT: return "invalid argument";
        case ADACOMP_ERR_UNSUPPORTED_BIN: return "unsupported bin length (1..32768)";
        case ADACOMP_ERR_MISALIGNED: return "misaligned segment offset or buffer";
        case ADACOMP_ERR_OVERLAP: return "segments overlap";
        case ADACOMP_ERR_CAPACITY: return "buffer smaller than the plan requires";
        case ADACOMP_ERR_HIP: return "HIP runtime error";
        case ADACOMP_ERR_TOO_LARGE: return "segment table too large";
        case ADACOMP_ERR_SCRATCH_LIMIT: return "plan workspace larger than the no-alloc scratch";
        default: return "unknown status";
    }
}

int adacomp_plan_query(const adacomp_segment* segs, uint32_t nseg, adacomp_plan_info* info) {
    if (info == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    try {
        Layout L;
        const int st = adacomp::build_layout(segs, nseg, L);
        if (st != ADACOMP_OK) return st;
        adacomp::fill_info(L, adacomp::choose_finish(L, 0u), info);
        return ADACOMP_OK;
    } catch (...) {
        return ADACOMP_ERR_INVALID_ARGUMENT;
    }
}

int adacomp_plan_create(const adacomp_segment* segs, uint32_t nseg, adacomp_plan** out) {
    return adacomp_plan_create_ex(segs, nseg, 0u, out);
}

int adacomp_plan_create_ex(const adacomp_segment* segs, uint32_t nseg, uint32_t plan_flags,
                           adacomp_plan** out) {
    if (out == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    const uint32_t finish_flags = plan_flags & ~ADACOMP_PLAN_DECODE_RECORDS;
    if (finish_flags != 0u && finish_flags != ADACOMP_PLAN_SEPARATE_FINISH &&
        finish_flags != ADACOMP_PLAN_SINGLE_LAUNCH)
        return ADACOMP_ERR_INVALID_ARGUMENT;
    adacomp_plan* p = nullptr;
    try {
        p = new adacomp_plan();
        int st = adacomp::build_layout(segs, nseg, p->L);
        if (st != ADACOMP_OK) {
            delete p;
            return st;
        }
        const Layout& L = p->L;
        // Launch limits: total work-items of one launch must fit in 32 bits.
        bool too_large = L.ct.ntiles * 256ull >= (uint64_t(1) << 32) ||
                         L.ct.nchunks * 256ull >= (uint64_t(1) << 32) ||
                         L.dt.nchunks * 256ull >= (uint64_t(1) << 32);
        for (int v = 0; v < adacomp::kVariants; ++v)
            too_large |= L.ct.by_variant[v].size() * uint64_t(adacomp::kVarThreads[v]) >=
                         (uint64_t(1) << 32);
        for (int v = 0; v < adacomp::kDecVariants; ++v)
            too_large |= L.dt.by_variant[v].size() * uint64_t(adacomp::kDecThreads[v]) >=
                         (uint64_t(1) << 32);
        if (too_large) {
            delete p;
            return ADACOMP_ERR_TOO_LARGE;
        }
        if (hipGetDevice(&p->device) != hipSuccess) {
            delete p;
            return ADACOMP_ERR_HIP;
        }
        // One device allocation holds every table.
        std::vector<uint8_t> host;
        auto put = [&host](const void* src, uint64_t bytes) {
            const uint64_t at = host.size();
            host.resize(adacomp::round_up(at + bytes + 4, 256), 0);
            if (bytes) std::memcpy(host.data() + at, src, bytes);
            return at;
        };
        struct TilingOffsets {
            uint64_t ts, v[adacomp::kVariants], ctb, cs;
        };
        auto put_tiling = [&](const adacomp::Tiling& T) {
            TilingOffsets o{};
            o.ts = put(T.tile_seg.data(), 4 * T.tile_seg.size());
            for (int v = 0; v < adacomp::kVariants; ++v)
                o.v[v] = put(T.by_variant[v].data(), 4 * T.by_variant[v].size());
            o.ctb = put(T.chunk_tile_begin.data(), 4 * T.chunk_tile_begin.size());
            o.cs = put(T.chunk_seg.data(), 4 * T.chunk_seg.size());
            return o;
        };
        const uint64_t o_segs = put(L.segs.data(), sizeof(SegDev) * L.nseg);
        const TilingOffsets oc = put_tiling(L.ct), od = put_tiling(L.dt);
        uint64_t o_cchunks = 0;
        {
            std::vector<adacomp::CountChunk> cc(L.dt.nchunks);
            for (uint64_t c = 0; c < L.dt.nchunks; ++c) {
                const SegDev& sg = L.segs[L.dt.chunk_seg[c]];
                adacomp::CountChunk& x = cc[c];
                x.count_off = sg.count_off;
                x.numel = sg.numel;
                x.tile0 = L.dt.chunk_tile_begin[c];
                x.ntiles = L.dt.chunk_tile_begin[c + 1] - x.tile0;
                x.first_bin = (x.tile0 - sg.dt.tile_begin) * sg.dt.bpt;
                x.bpt = sg.dt.bpt;
                x.nbins = sg.nbins;
                x.wb = sg.wb;
                x.lt = sg.lt;
            }
            o_cchunks = put(cc.data(), sizeof(adacomp::CountChunk) * cc.size());
        }
        uint64_t o_desc[adacomp::kDecVariants];
        for (int v = 0; v < adacomp::kDecVariants; ++v) {
            const std::vector<adacomp::DecDesc> d = adacomp::decode_descs(L, v);
            o_desc[v] = put(d.data(), sizeof(adacomp::DecDesc) * d.size());
        }
        p->finish = adacomp::choose_finish(L, finish_flags);
        uint64_t o_t0 = 0;
        if (adacomp::uses_small_tables(p->finish)) {
            std::vector<uint32_t> t0(L.ct.ntiles);
            for (uint64_t t = 0; t < L.ct.ntiles; ++t) {
                const SegDev& sg = L.segs[L.ct.tile_seg[t]];
                t0[t] = static_cast<uint32_t>(adacomp::tile_geom(sg, sg.ct, uint32_t(t)).t0);
            }
            o_t0 = put(t0.data(), 4 * t0.size());
        }
        if (hipMalloc(&p->dmem, host.size()) != hipSuccess) {
            p->dmem = nullptr;
            delete p;
            return ADACOMP_ERR_HIP;
        }
        if (hipMemcpy(p->dmem, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipFree(p->dmem);
            delete p;
            return ADACOMP_ERR_HIP;
        }
        uint8_t* base = static_cast<uint8_t*>(p->dmem);
        p->d_segs = reinterpret_cast<SegDev*>(base + o_segs);
        p->d_cchunks = reinterpret_cast<adacomp::CountChunk*>(base + o_cchunks);
        auto bind = [base](DevTiling& d, const TilingOffsets& o) {
            d.tile_seg = reinterpret_cast<uint32_t*>(base + o.ts);
            for (int v = 0; v < adacomp::kVariants; ++v)
                d.vtiles[v] = reinterpret_cast<uint32_t*>(base + o.v[v]);
            d.chunk_tile_begin = reinterpret_cast<uint32_t*>(base + o.ctb);
            d.chunk_seg = reinterpret_cast<uint32_t*>(base + o.cs);
        };
        bind(p->dct, oc);
        bind(p->ddt, od);
        for (int v = 0; v < adacomp::kDecVariants; ++v)
            p->ddesc[v] = reinterpret_cast<adacomp::DecDesc*>(base + o_desc[v]);
        if (adacomp::uses_small_tables(p->finish))
            p->tile_t0 = reinterpret_cast<uint32_t*>(base + o_t0);
        // Per tile: bin maxima, bin boundaries, and for hard local selection
        // the first index of each bin's maximum.
        for (int v = 0; v < adacomp::kVariants; ++v)
            p->tile_lds_words[v] = (L.has_ls ? 3 : 2) * L.ct.max_bpt[v] + 1;
        p->small_lds_bytes = static_cast<uint32_t>(
            adacomp::round_up(adacomp::small_lds_bytes(L.ct.ntiles, L.ct.nchunks, L.nseg), 8));
        p->single_lds_bytes = std::max<uint32_t>(
            4 * std::max(L.ct.by_variant[0].empty() ? 0u : p->tile_lds_words[0],
                         L.ct.by_variant[1].empty() ? 0u : p->tile_lds_words[1]),
            p->small_lds_bytes);
        p->chunk_lds_bytes = static_cast<uint32_t>(
            adacomp::round_up(adacomp::chunk_finish_lds_bytes(L.ct.nchunks, L.nseg), 8));
        p->sum_kernel = L.dt.by_variant[0].size() >= kSumKernelMinTiles;
        for (const SegDev& sg : L.segs)
            if (sg.dt.variant == 0u && sg.wb != 2u) p->sum_kernel = false;
        if (plan_flags & ADACOMP_PLAN_DECODE_RECORDS) p->sum_kernel = true;
        if (L.dt.by_variant[0].empty()) p->sum_kernel = false;
        for (const SegDev& sg : L.segs) {
            if (uint64_t(sg.dt.bpt) * sg.wb > kCountBatchMinBytes && L.dt.ntiles >= kSumKernelMinTiles)
                p->count_batched = true;
            if (sg.dt.variant == 0u && sg.wb == 1u) p->dense_words = true;
        }
        *out = p;
        return ADACOMP_OK;
    } catch (...) {
        if (p) {
            if (p->dmem) (void)hipFree(p->dmem);
            delete p;
        }
        return ADACOMP_ERR_INVALID_ARGUMENT;
    }
}

int adacomp_plan_destroy(adacomp_plan* plan) {
    if (plan == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    int st = ADACOMP_OK;
    if (plan->dmem && hipFree(plan->dmem) != hipSuccess) st = ADACOMP_ERR_HIP;
    delete plan;
    return st;
}

int adacomp_plan_get_info(const adacomp_plan* plan, adacomp_plan_info* info) {
    if (plan == nullptr || info == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    adacomp::fill_info(plan->L, plan->finish, info);
    return ADACOMP_OK;
}

int adacomp_compress_timed(const adacomp_plan* plan, float* residue, const float* dW,
                           uint64_t n_elems, void* msg, uint64_t msg_bytes, void* ws,
                           uint64_t ws_bytes, float* bin_max_out, void* stream_,
                           adacomp_timer* timer) {
    if (plan == nullptr || residue == nullptr || dW == nullptr || msg == nullptr || ws == nullptr)
        return ADACOMP_ERR_INVALID_ARGUMENT;
    const Layout& L = plan->L;
    if (!aligned16(residue) || !aligned16(dW) || !aligned16(msg) || !aligned16(ws))
        return ADACOMP_ERR_MISALIGNED;
    if (bin_max_out != nullptr && (reinterpret_cast<uintptr_t>(bin_max_out) & 3u) != 0)
        return ADACOMP_ERR_MISALIGNED;
    if (n_elems < L.span || msg_bytes < L.capacity || ws_bytes < L.ws_compress)
        return ADACOMP_ERR_CAPACITY;
    {
        // a fixed array: this check allocates nothing (adacomp_compress_noalloc)
        const Range r[5] = {range_of(residue, 4 * L.span), range_of(dW, 4 * L.span),
                            range_of(msg, L.capacity), range_of(ws, L.ws_compress),
                            range_of(bin_max_out, bin_max_out ? 4 * L.total_bins : 0)};
        const int nr = bin_max_out ? 5 : 4;
        for (int i = 0; i < nr; ++i)
            for (int j = i + 1; j < nr; ++j)
                if (overlaps(r[i], r[j])) return ADACOMP_ERR_INVALID_ARGUMENT;
    }
    int st = check_device(plan);
    if (st != ADACOMP_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);

    uint8_t* w8 = static_cast<uint8_t*>(ws);
    uint32_t* stage = reinterpret_cast<uint32_t*>(w8 + L.ws_stage);
    uint32_t* tile_cnt = reinterpret_cast<uint32_t*>(w8 + L.ws_tile_cnt);
    double* tile_gsum = reinterpret_cast<double*>(w8 + L.ws_tile_gsum);
    uint32_t* tile_off = reinterpret_cast<uint32_t*>(w8 + L.ws_tile_off);
    uint32_t* chunk_cnt = reinterpret_cast<uint32_t*>(w8 + L.ws_chunk_cnt);
    double* chunk_gsum = reinterpret_cast<double*>(w8 + L.ws_chunk_gsum);
    uint32_t* chunk_base = reinterpret_cast<uint32_t*>(w8 + L.ws_chunk_base);
    float* seg_s = reinterpret_cast<float*>(w8 + L.ws_seg_s);
    uint32_t* seg_nsurv = reinterpret_cast<uint32_t*>(w8 + L.ws_seg_nsurv);
    uint64_t* seg_eoff = reinterpret_cast<uint64_t*>(w8 + L.ws_seg_eoff);
    uint64_t* seg_sbase = reinterpret_cast<uint64_t*>(w8 + L.ws_seg_sbase);
    uint8_t* m8 = static_cast<uint8_t*>(msg);

    CallTimer tm(timer, stream, ADACOMP_STAGE_COMPRESS_CALL);
    adacomp::SmallArgs sa{};
    if (adacomp::uses_small_tables(plan->finish)) {
        sa.segs = plan->d_segs;
        sa.tile_seg = plan->dct.tile_seg;
        sa.tile_t0 = plan->tile_t0;
        sa.vtiles0 = plan->dct.vtiles[0];
        sa.vtiles1 = plan->dct.vtiles[1];
        sa.chunk_tile_begin = plan->dct.chunk_tile_begin;
        sa.residue = residue;
        sa.dW = dW;
        sa.msg = m8;
        sa.stage = stage;
        sa.tile_cnt = tile_cnt;
        sa.tile_gsum = tile_gsum;
        sa.bin_max_out = bin_max_out;
        sa.sync = reinterpret_cast<uint64_t*>(w8 + L.ws_sync);
        sa.entries_begin = L.entries_begin;
        sa.n0 = static_cast<uint32_t>(L.ct.by_variant[0].size());
        sa.ntiles = static_cast<uint32_t>(L.ct.ntiles);
        sa.nchunks = static_cast<uint32_t>(L.ct.nchunks);
        sa.nseg = L.nseg;
        sa.plan_hash = L.plan_hash;
    }
    if (plan->finish == adacomp::Finish::kSingle) {
        hipLaunchKernelGGL(adacomp::k_compress_single, dim3(sa.ntiles), dim3(256),
                           plan->single_lds_bytes, stream, sa);
        if ((st = launch_status()) != ADACOMP_OK) return st;
        tm.finish();
        return ADACOMP_OK;
    }
    {
        for (int v = 0; v < adacomp::kVariants; ++v) {
            if (L.ct.by_variant[v].empty()) continue;
            hipError_t e;
            if (v == 0)
                e = adacomp::launch_tile_pass<0>(plan, stream, residue, dW, m8, stage, tile_cnt,
                                                 tile_gsum, bin_max_out);
            else if (v == 1)
                e = adacomp::launch_tile_pass<1>(plan, stream, residue, dW, m8, stage, tile_cnt,
                                                 tile_gsum, bin_max_out);
            else
                e = adacomp::launch_tile_pass<2>(plan, stream, residue, dW, m8, stage, tile_cnt,
                                                 tile_gsum, bin_max_out);
            if (e != hipSuccess) return ADACOMP_ERR_HIP;
        }
        tm.mark(ADACOMP_STAGE_TILE_PASS);
    }
    if (plan->finish == adacomp::Finish::kSmall) {
        hipLaunchKernelGGL(adacomp::k_finish_small, dim3(encode_blocks(L)), dim3(256),
                           plan->small_lds_bytes, stream, sa);
        if ((st = launch_status()) != ADACOMP_OK) return st;
        tm.mark(ADACOMP_STAGE_ENCODE);
        tm.finish();
        return ADACOMP_OK;
    }
    {
        hipLaunchKernelGGL(adacomp::k_chunk_scan, dim3(static_cast<uint32_t>(L.ct.nchunks)), dim3(256),
                           0, stream, plan->dct.chunk_tile_begin, tile_cnt, tile_gsum, tile_off,
                           chunk_cnt, chunk_gsum);
        if ((st = launch_status()) != ADACOMP_OK) return st;
        tm.mark(ADACOMP_STAGE_CHUNK_SCAN);
    }
    if (plan->finish == adacomp::Finish::kChunks) {
        adacomp::ChunkFinishArgs ca{};
        ca.segs = plan->d_segs;
        ca.tile_seg = plan->dct.tile_seg;
        ca.stage = stage;
        ca.tile_cnt = tile_cnt;
        ca.tile_off = tile_off;
        ca.chunk_cnt = chunk_cnt;
        ca.chunk_gsum = chunk_gsum;
        ca.msg = m8;
        ca.residue = residue;
        ca.entries_begin = L.entries_begin;
        ca.nchunks = static_cast<uint32_t>(L.ct.nchunks);
        ca.nseg = L.nseg;
        ca.ntiles = static_cast<uint32_t>(L.ct.ntiles);
        ca.plan_hash = L.plan_hash;
        hipLaunchKernelGGL(adacomp::k_finish_chunks, dim3(encode_blocks(L)), dim3(256),
                           plan->chunk_lds_bytes, stream, ca);
        if ((st = launch_status()) != ADACOMP_OK) return st;
        tm.mark(ADACOMP_STAGE_ENCODE);
        tm.finish();
        return ADACOMP_OK;
    }
    {
        hipLaunchKernelGGL(adacomp::k_finalize, dim3(1), dim3(256), 0, stream, plan->d_segs, L.nseg,
                           L.plan_hash, L.entries_begin, chunk_cnt, chunk_gsum, chunk_base, seg_s,
                           seg_nsurv, seg_eoff, seg_sbase, m8);
        if ((st = launch_status()) != ADACOMP_OK) return st;
        tm.mark(ADACOMP_STAGE_FINALIZE);
    }
    {
        hipLaunchKernelGGL(adacomp::k_encode, dim3(encode_blocks(L)), dim3(256), 0, stream,
                           plan->d_segs, L.nseg, plan->dct.tile_seg, stage, tile_cnt, tile_off,
                           chunk_base, seg_s, seg_eoff, seg_sbase, m8, residue,
                           static_cast<uint32_t>(L.ct.ntiles));
        if ((st = launch_status()) != ADACOMP_OK) return st;
        tm.mark(ADACOMP_STAGE_ENCODE);
    }
    tm.finish();
    return ADACOMP_OK;
}

int adacomp_compress(const adacomp_plan* plan, float* residue, const float* dW, uint64_t n_elems,
                     void* msg, uint64_t msg_bytes, void* ws, uint64_t ws_bytes,
                     float* bin_max_out, void* stream) {
    return adacomp_compress_timed(plan, residue, dW, n_elems, msg, msg_bytes, ws, ws_bytes,
                                  bin_max_out, stream, nullptr);
}

}  // extern "C"

// Workspace of adacomp_compress_noalloc: a file-scope device array, one copy
// per GPU.  Host code never uses its name as an address (on the host it is
// only a stand-in); the device address comes from hipGetSymbolAddress, once
// per device, and is kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[ADACOMP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> scratch_ptr[kScratchDevices];

// The current device's copy of `scratch`, looked up on the first call on
// that device (with it current) and kept for the process.
int scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return ADACOMP_ERR_HIP;
    if (dev < 0 || dev >= kScratchDevices) return ADACOMP_ERR_INVALID_ARGUMENT;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return ADACOMP_ERR_HIP;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return ADACOMP_OK;
}
}  // namespace

extern "C" {

int adacomp_compress_noalloc(const adacomp_plan* plan, float* residue, const float* dW,
                             uint64_t n_elems, void* msg, uint64_t msg_bytes, float* bin_max_out,
                             void* stream) {
    if (plan == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    if (plan->L.ws_compress > ADACOMP_NOALLOC_SCRATCH_BYTES) return ADACOMP_ERR_SCRATCH_LIMIT;
    int st = check_device(plan);
    if (st != ADACOMP_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != ADACOMP_OK) return st;
    return adacomp_compress_timed(plan, residue, dW, n_elems, msg, msg_bytes, ws,
                                  ADACOMP_NOALLOC_SCRATCH_BYTES, bin_max_out, stream, nullptr);
}

}  // extern "C"

namespace {

// Workspace of decode + SGD: the decode workspace, then (plans with bins
// longer than 4093) a dense float32 scratch for those tiles' sums.
struct SgdLayout {
    uint64_t decode_bytes, scratch, total;
};
SgdLayout sgd_layout(const Layout& L, uint32_t K) {
    SgdLayout o{};
    const uint64_t d = std::max<uint64_t>(decode_layout(L, K).total, L.dws_fixed + uint64_t(K) * L.dws_per_msg);
    o.decode_bytes = d;
    o.scratch = adacomp::round_up(d, adacomp::kAlign);
    o.total = o.scratch + (L.dt.by_variant[1].empty() ? 0 : 4 * L.span);
    return o;
}

// Shared by decode_accumulate (opt == kOptNone, out) and decode fused with
// an optimizer step (op.w, op.m and, for Adam, op.v).
int decode_impl(const adacomp_plan* plan, const void* const* msgs, uint32_t K, float* out,
                int accumulate, int opt, adacomp::OptParams op, uint64_t n_elems, void* ws,
                uint64_t ws_bytes, void* stream_, adacomp_timer* timer, int call_stage) {
    const bool fused = opt != adacomp::kOptNone;
    if (plan == nullptr || msgs == nullptr || ws == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    if (K == 0 || K > ADACOMP_MAX_MESSAGES) return ADACOMP_ERR_INVALID_ARGUMENT;
    if (accumulate != 0 && accumulate != 1) return ADACOMP_ERR_INVALID_ARGUMENT;
    const Layout& L = plan->L;
    const DecodeLayout D = decode_layout(L, K);
    const SgdLayout S = sgd_layout(L, K);
    std::vector<Range> dense;   // the dense buffers written
    if (!fused) {
        if (out == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
        if (!aligned16(out)) return ADACOMP_ERR_MISALIGNED;
        dense.push_back(range_of(out, 4 * L.span));
    } else {
        float* st_bufs[3] = {op.w, op.m, opt == adacomp::kOptAdam ? op.v : op.w};
        for (int i = 0; i < (opt == adacomp::kOptAdam ? 3 : 2); ++i) {
            if (st_bufs[i] == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
            if (!aligned16(st_bufs[i])) return ADACOMP_ERR_MISALIGNED;
            dense.push_back(range_of(st_bufs[i], 4 * L.span));
        }
    }
    if (!aligned16(ws)) return ADACOMP_ERR_MISALIGNED;
    const uint64_t need = fused ? S.total : std::max<uint64_t>(D.total, L.dws_fixed + uint64_t(K) * L.dws_per_msg);
    if (n_elems < L.span || ws_bytes < need) return ADACOMP_ERR_CAPACITY;
    const Range rw = range_of(ws, need);
    for (size_t i = 0; i < dense.size(); ++i) {
        if (overlaps(dense[i], rw)) return ADACOMP_ERR_INVALID_ARGUMENT;
        for (size_t j = i + 1; j < dense.size(); ++j)
            if (overlaps(dense[i], dense[j])) return ADACOMP_ERR_INVALID_ARGUMENT;
    }
    adacomp::MsgPtrs mp{};
    for (uint32_t k = 0; k < K; ++k) {
        if (msgs[k] == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
        if (!aligned16(msgs[k])) return ADACOMP_ERR_MISALIGNED;
        // entry records hold 48-bit addresses
        if (reinterpret_cast<uintptr_t>(msgs[k]) + L.capacity >= (uint64_t(1) << 48))
            return ADACOMP_ERR_INVALID_ARGUMENT;
        const Range rm = range_of(msgs[k], 32 + 16 * uint64_t(L.nseg));
        if (overlaps(rm, rw)) return ADACOMP_ERR_INVALID_ARGUMENT;
        for (const Range& r : dense)
            if (overlaps(rm, r)) return ADACOMP_ERR_INVALID_ARGUMENT;
        mp.p[k] = static_cast<const uint8_t*>(msgs[k]);
    }
    int st = check_device(plan);
    if (st != ADACOMP_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);

    uint8_t* w8 = static_cast<uint8_t*>(ws);
    adacomp::DecodeWs dw;
    dw.status = reinterpret_cast<uint32_t*>(w8 + D.status);
    dw.dcnt = reinterpret_cast<uint32_t*>(w8 + D.dcnt);
    dw.doff = reinterpret_cast<uint32_t*>(w8 + D.doff);
    dw.dchunk_cnt = reinterpret_cast<uint32_t*>(w8 + D.dchunk_cnt);
    dw.dchunk_base = reinterpret_cast<uint32_t*>(w8 + D.dchunk_base);
    dw.dseg_s = reinterpret_cast<float*>(w8 + D.dseg_s);
    dw.dseg_eoff = reinterpret_cast<uint64_t*>(w8 + D.dseg_eoff);
    dw.dvalid = reinterpret_cast<uint32_t*>(w8 + D.dvalid);
    dw.drec = reinterpret_cast<uint64_t*>(w8 + D.drec);
    const uint32_t DT = static_cast<uint32_t>(L.dt.ntiles), DC = static_cast<uint32_t>(L.dt.nchunks);
    float* sums = out;   // where long-bin tiles accumulate
    if (fused) {
        sums = reinterpret_cast<float*>(w8 + S.scratch);
        accumulate = 0;
    }

    adacomp::MsgGeom geo{};
    geo.nseg = L.nseg;
    geo.plan_hash = L.plan_hash;
    geo.entries_begin = L.entries_begin;
    geo.capacity = L.capacity;

    // The plain sum of at most 16 messages from +0 over many LDS tiles of 16-bit words
    // (sparse messages) takes the two-round-trip kernel; everything else (more messages,
    // out += sum, an optimizer step, 8-bit words, smaller tables) k_decode_tiles.
    const uint32_t ps0 = L.dt.max_bpt[0] + 1;
    const bool plain_sum = plan->sum_kernel && !fused && accumulate == 0 &&
                           adacomp::decode_tiles_group(K, ps0) == K;
    CallTimer tm(timer, stream, call_stage);
    {
        if (plan->count_batched)
            hipLaunchKernelGGL(adacomp::k_decode_count<8>, dim3(DC, K), dim3(256), 0, stream, mp,
                               plan->d_cchunks, DT, DC, geo, dw);
        else
            hipLaunchKernelGGL(adacomp::k_decode_count<0>, dim3(DC, K), dim3(256), 0, stream, mp,
                               plan->d_cchunks, DT, DC, geo, dw);
        if ((st = launch_status()) != ADACOMP_OK) return st;
        tm.mark(ADACOMP_STAGE_DECODE_COUNT);
    }
    {
        hipLaunchKernelGGL(adacomp::k_decode_base, dim3(K), dim3(256), 0, stream, mp, K,
                           plan->d_segs, geo, DC, dw);
        if ((st = launch_status()) != ADACOMP_OK) return st;
        if (plain_sum) {   // the LDS tiles' entry records for k_decode_tiles_sum
            const uint32_t P = static_cast<uint32_t>(L.dt.by_variant[0].size());
            hipLaunchKernelGGL(adacomp::k_decode_records, dim3((P + 255) / 256), dim3(256), 0, stream,
                               mp, K, plan->ddesc[0], P, DT, DC, L.nseg, dw);
            if ((st = launch_status()) != ADACOMP_OK) return st;
        }
        tm.mark(ADACOMP_STAGE_DECODE_BASE);
    }
    {
        for (int v = 0; v < adacomp::kDecVariants; ++v) {
            const uint32_t n = static_cast<uint32_t>(L.dt.by_variant[v].size());
            if (n == 0) continue;
            const uint32_t ps = L.dt.max_bpt[v] + 1;
            const uint32_t KG = adacomp::decode_group(K, ps);
            if (v == 0) {   // tiles of at most 4096 elements: bits per message, then ordered sums
                const uint32_t acc_words = L.dt.max_span_vecs[0] * 4;
                const uint32_t kg = adacomp::decode_tiles_group(K, ps);
                const bool sep = kg < K || (accumulate != 0 && !fused);
                // The bin-start table: plain decodes of tables of 8-bit words only; on smaller tables (fewer
                // than kSumKernelMinTiles LDS decode tiles) with kTblBytes of its own, on larger
                // ones in the place of the bin prefixes alone (no LDS beyond them).
                const uint32_t tblw = !plan->dense_words || opt != adacomp::kOptNone ? 0u
                                      : n < kSumKernelMinTiles
                                          ? std::max(adacomp::kTblBytes / 4u, adacomp::decode_tiles_pref_words(kg, ps))
                                          : adacomp::decode_tiles_pref_words(kg, ps);
                const uint32_t lds = adacomp::decode_tiles_lds_bytes(acc_words, K, kg, ps, sep, tblw);
                float* dst = fused ? nullptr : out;
                const int acc = fused ? 0 : accumulate;
#define ADACOMP_TILES(SEP, OPT)                                                                    \
    hipLaunchKernelGGL((adacomp::k_decode_tiles<SEP, OPT, false>), dim3(n), dim3(256), lds, stream, mp, \
                       K, kg, ps, plan->ddesc[0], DT, DC, L.nseg, dw, dst, acc, acc_words, op, 0u)
#define ADACOMP_TILES_TBL(SEP)                                                                     \
    hipLaunchKernelGGL((adacomp::k_decode_tiles<SEP, adacomp::kOptNone, true>), dim3(n), dim3(256), lds, \
                       stream, mp, K, kg, ps, plan->ddesc[0], DT, DC, L.nseg, dw, dst, acc, acc_words, op, tblw)
                if (plain_sum) {
                    hipLaunchKernelGGL(adacomp::k_decode_tiles_sum, dim3(n), dim3(256),
                                       adacomp::decode_sum_lds_bytes(acc_words, K, ps), stream, mp, K,
                                       ps, plan->ddesc[0], L.nseg, dw, out, acc_words);
                } else if (opt == adacomp::kOptSgd) {
                    if (sep) ADACOMP_TILES(true, adacomp::kOptSgd);
                    else ADACOMP_TILES(false, adacomp::kOptSgd);
                } else if (opt == adacomp::kOptAdam) {
                    if (sep) ADACOMP_TILES(true, adacomp::kOptAdam);
                    else ADACOMP_TILES(false, adacomp::kOptAdam);
                } else if (tblw != 0u) {
                    if (sep) ADACOMP_TILES_TBL(true);
                    else ADACOMP_TILES_TBL(false);
                } else {
                    if (sep) ADACOMP_TILES(true, adacomp::kOptNone);
                    else ADACOMP_TILES(false, adacomp::kOptNone);
                }
#undef ADACOMP_TILES
#undef ADACOMP_TILES_TBL
            } else if (long_decode_in_lds(L, K, KG, ps, opt)) {
                // long bins, the whole tile accumulated in LDS (one 1024-thread workgroup per
                // CU) and written once, or stepped by the optimizer
                const uint32_t acc_words = L.dt.max_span_vecs[1] * 4;
                const uint32_t lds = adacomp::decode_lds_bytes(acc_words, K, KG, ps, 16);
                if (opt == adacomp::kOptSgd)
                    hipLaunchKernelGGL((adacomp::k_decode_apply<1024, true, adacomp::kOptSgd>), dim3(n),
                                       dim3(1024), lds, stream, mp, K, KG, ps, plan->ddesc[1], DT, DC,
                                       L.nseg, dw, nullptr, 0, acc_words, op);
                else if (opt == adacomp::kOptAdam)
                    hipLaunchKernelGGL((adacomp::k_decode_apply<1024, true, adacomp::kOptAdam>), dim3(n),
                                       dim3(1024), lds, stream, mp, K, KG, ps, plan->ddesc[1], DT, DC,
                                       L.nseg, dw, nullptr, 0, acc_words, op);
                else
                    hipLaunchKernelGGL((adacomp::k_decode_apply<1024, true>), dim3(n), dim3(1024), lds,
                                       stream, mp, K, KG, ps, plan->ddesc[1], DT, DC, L.nseg, dw, out,
                                       accumulate, acc_words, op);
            } else {   // long bins accumulated in place: in out, or in the scratch for an optimizer step
                const uint32_t lds = adacomp::decode_lds_bytes(0, K, KG, ps, 16);
                hipLaunchKernelGGL((adacomp::k_decode_apply<1024, false>), dim3(n), dim3(1024), lds,
                                   stream, mp, K, KG, ps, plan->ddesc[1], DT, DC, L.nseg, dw, sums,
                                   accumulate, 0u, op);
                if (launch_status() == ADACOMP_OK) {
                    if (opt == adacomp::kOptSgd)
                        hipLaunchKernelGGL(adacomp::k_opt_tiles<adacomp::kOptSgd>, dim3(n), dim3(256), 0,
                                           stream, plan->ddesc[1], sums, op);
                    else if (opt == adacomp::kOptAdam)
                        hipLaunchKernelGGL(adacomp::k_opt_tiles<adacomp::kOptAdam>, dim3(n), dim3(256),
                                           0, stream, plan->ddesc[1], sums, op);
                }
            }
            if ((st = launch_status()) != ADACOMP_OK) return st;
        }
        tm.mark(ADACOMP_STAGE_DECODE_APPLY);
    }
    tm.finish();
    return ADACOMP_OK;
}

}  // namespace

extern "C" {

int adacomp_decode_accumulate_timed(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                                    float* out, uint64_t n_elems, int accumulate, void* ws,
                                    uint64_t ws_bytes, void* stream, adacomp_timer* timer) {
    return decode_impl(plan, msgs, K, out, accumulate, adacomp::kOptNone, adacomp::OptParams{},
                       n_elems, ws, ws_bytes, stream, timer, ADACOMP_STAGE_DECODE_CALL);
}

int adacomp_decode_accumulate(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                              float* out, uint64_t n_elems, int accumulate, void* ws,
                              uint64_t ws_bytes, void* stream) {
    return adacomp_decode_accumulate_timed(plan, msgs, K, out, n_elems, accumulate, ws, ws_bytes,
                                           stream, nullptr);
}

int adacomp_decode_sgd_workspace_bytes(const adacomp_plan* plan, uint32_t K, uint64_t* bytes) {
    if (plan == nullptr || bytes == nullptr || K == 0 || K > ADACOMP_MAX_MESSAGES)
        return ADACOMP_ERR_INVALID_ARGUMENT;
    *bytes = sgd_layout(plan->L, K).total;
    return ADACOMP_OK;
}

int adacomp_decode_sgd_timed(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                             float* weights, float* momentum, uint64_t n_elems,
                             const adacomp_sgd* sgd, void* ws, uint64_t ws_bytes, void* stream,
                             adacomp_timer* timer) {
    if (sgd == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    adacomp::OptParams op{};
    op.lr = sgd->lr;
    op.beta1 = sgd->momentum;
    op.weight_decay = sgd->weight_decay;
    op.scale = sgd->scale;
    op.w = weights;
    op.m = momentum;
    return decode_impl(plan, msgs, K, nullptr, 0, adacomp::kOptSgd, op, n_elems, ws, ws_bytes,
                       stream, timer, ADACOMP_STAGE_DECODE_SGD_CALL);
}

int adacomp_decode_adam_timed(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                              float* weights, float* m, float* v, uint64_t n_elems,
                              const adacomp_adam* adam, void* ws, uint64_t ws_bytes, void* stream,
                              adacomp_timer* timer) {
    if (adam == nullptr || adam->step == 0) return ADACOMP_ERR_INVALID_ARGUMENT;
    adacomp::OptParams op{};
    op.lr = adam->lr;
    op.beta1 = adam->beta1;
    op.beta2 = adam->beta2;
    op.eps = adam->eps;
    op.weight_decay = adam->weight_decay;
    op.scale = adam->scale;
    // bias corrections in double, rounded once; 1 - beta as float operations
    op.c1 = static_cast<float>(1.0 - std::pow(static_cast<double>(adam->beta1), static_cast<double>(adam->step)));
    op.c2 = static_cast<float>(1.0 - std::pow(static_cast<double>(adam->beta2), static_cast<double>(adam->step)));
    op.omb1 = 1.0f - adam->beta1;
    op.omb2 = 1.0f - adam->beta2;
    op.w = weights;
    op.m = m;
    op.v = v;
    return decode_impl(plan, msgs, K, nullptr, 0, adacomp::kOptAdam, op, n_elems, ws, ws_bytes,
                       stream, timer, ADACOMP_STAGE_DECODE_ADAM_CALL);
}

int adacomp_decode_adam(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                        float* weights, float* m, float* v, uint64_t n_elems,
                        const adacomp_adam* adam, void* ws, uint64_t ws_bytes, void* stream) {
    return adacomp_decode_adam_timed(plan, msgs, K, weights, m, v, n_elems, adam, ws, ws_bytes,
                                     stream, nullptr);
}

int adacomp_decode_sgd(const adacomp_plan* plan, const void* const* msgs, uint32_t K,
                       float* weights, float* momentum, uint64_t n_elems, const adacomp_sgd* sgd,
                       void* ws, uint64_t ws_bytes, void* stream) {
    return adacomp_decode_sgd_timed(plan, msgs, K, weights, momentum, n_elems, sgd, ws, ws_bytes,
                                    stream, nullptr);
}

int adacomp_timer_create(adacomp_timer** timer) {
    if (timer == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    *timer = new (std::nothrow) adacomp_timer();
    return *timer ? ADACOMP_OK : ADACOMP_ERR_INVALID_ARGUMENT;
}

int adacomp_timer_reset(adacomp_timer* timer) {
    if (timer == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    int st = ADACOMP_OK;
    for (auto& c : timer->calls) {
        if (hipEventSynchronize(c.ev.back()) != hipSuccess) st = ADACOMP_ERR_HIP;
        for (hipEvent_t e : c.ev) (void)hipEventDestroy(e);
    }
    timer->calls.clear();
    for (int i = 0; i < ADACOMP_NUM_STAGES; ++i) {
        timer->ms[i] = 0.0;
        timer->n[i] = 0;
    }
    return st;
}

int adacomp_timer_destroy(adacomp_timer* timer) {
    if (timer == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    const int st = adacomp_timer_reset(timer);
    delete timer;
    return st;
}

int adacomp_timer_read(adacomp_timer* timer, double* ms, uint64_t* launches, uint32_t nstages) {
    if (timer == nullptr || ms == nullptr || launches == nullptr) return ADACOMP_ERR_INVALID_ARGUMENT;
    // Each call is added whole or not at all; a call whose events cannot be
    // read is dropped (the calls before it stay counted), so no call is
    // counted twice.
    size_t done = 0;
    int st = ADACOMP_OK;
    std::vector<float> t;
    for (; done < timer->calls.size(); ++done) {
        adacomp_timer::Call& c = timer->calls[done];
        t.assign(c.stage.size() + 1, 0.f);
        bool ok = hipEventSynchronize(c.ev.back()) == hipSuccess;
        for (size_t i = 0; ok && i < c.stage.size(); ++i)
            ok = hipEventElapsedTime(&t[i], c.ev[i], c.ev[i + 1]) == hipSuccess;
        ok = ok && hipEventElapsedTime(&t.back(), c.ev.front(), c.ev.back()) == hipSuccess;
        if (ok) {
            for (size_t i = 0; i < c.stage.size(); ++i) {
                timer->ms[c.stage[i]] += t[i];
                timer->n[c.stage[i]] += 1;
            }
            timer->ms[c.whole] += t.back();
            timer->n[c.whole] += 1;
        }
        for (hipEvent_t e : c.ev) (void)hipEventDestroy(e);
        if (!ok) {
            st = ADACOMP_ERR_HIP;
            ++done;
            break;
        }
    }
    timer->calls.erase(timer->calls.begin(), timer->calls.begin() + static_cast<std::ptrdiff_t>(done));
    if (st != ADACOMP_OK) return st;
    for (uint32_t i = 0; i < nstages && i < ADACOMP_NUM_STAGES; ++i) {
        ms[i] = timer->ms[i];
        launches[i] = timer->n[i];
    }
    return ADACOMP_OK;
}

}  // extern "C"
