// HIP kernels of the AdaComp compressor and decode-accumulate for gfx950.
//
// Method: "AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
// page, definition paragraph and Mechanism claim on local-bin soft threshold
// and mean-g_max quantization (Algorithm 2); word widths from its Application
// claim (Table 2).
//
// The path is HBM-bandwidth bound (about 6 float32 operations per 12 bytes
// moved), so the kernels are built around coalesced 16-byte accesses, whole
// bins per workgroup and compaction in LDS; no matrix cores are involved.
//
// Compress, per call, four stream-ordered launches:
//   tile pass   (dense, one workgroup per tile of whole bins): reads residue
//               and dW once as float4, forms G and H, bin maxima by a
//               segmented wavefront max-scan plus LDS atomics, the survivor
//               test |H| >= g_max && G != 0, survivor ranks by ballot and
//               popcount, writes residue = G for every element, the bin's
//               count word into the message, and the tile's survivors as
//               (tile offset | sign, G) pairs to a staging area;
//   chunk scan  survivor offsets of tiles inside chunks of 1024 tiles and the
//               chunk's float64 sum of bin maxima, in a fixed order;
//   finalize    one workgroup: s per segment, entry region offsets, survivors
//               before each segment, message header, directory and padding;
//   encode      the survivors shared out evenly among wavefronts: entry words
//               into the message and the residue of each survivor,
//               G - sign(G) * s.
// Decode, per call, three launches: per-tile counts of every message, chunk
// bases and message validity, then the per-tile apply that sums the messages
// in order in LDS (large tiles: directly in out) and writes each tile once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace adacomp {

constexpr uint32_t kSentinel = 0xFFFFFFFFu;

#ifndef ADACOMP_NT_DW
#define ADACOMP_NT_DW 1
#endif
#ifndef ADACOMP_NT_R
#define ADACOMP_NT_R 1
#endif
#ifndef ADACOMP_NT_ST
#define ADACOMP_NT_ST 1
#endif

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming float4 access.  residue and dW are read once and the residue
// written once per call, so all three use non-temporal accesses (measured
// fastest on MI355X for this read-read-write stream).
template <bool NT>
__device__ __forceinline__ f32x4 load4(const float* p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return *reinterpret_cast<const f32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void store4(float* p, f32x4 v) {
    if (NT) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = v;
}

__device__ __forceinline__ uint64_t rup16(uint64_t x) { return (x + 15u) & ~uint64_t(15); }

__device__ __forceinline__ void put_word(uint8_t* p, uint32_t wb, uint32_t v) {
    if (wb == 1u) *p = static_cast<uint8_t>(v);
    else *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v);
}

__device__ __forceinline__ uint32_t get_word(const uint8_t* p, uint32_t wb) {
    return wb == 1u ? uint32_t(*p) : uint32_t(*reinterpret_cast<const uint16_t*>(p));
}

// ---------------------------------------------------------------------------
// Compress, dense tile pass.
// ---------------------------------------------------------------------------
constexpr uint32_t kNoKey = 0xFFFFFFFEu;   // never a bin index nor kSentinel

// DPP lane moves (VALU, no LDS round trip).  Lanes without a source, and
// lanes of rows masked off, receive `old`.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROWS, 0xf, false));
}
// lane l receives lane l+1 (wave_shl:1); lane 63 receives old
__device__ __forceinline__ uint32_t from_next_lane(uint32_t old, uint32_t v) { return dpp_u32<0x130>(old, v); }
// lane l receives lane l-1 (wave_shr:1); lane 0 receives old
__device__ __forceinline__ uint32_t from_prev_lane(uint32_t old, uint32_t v) { return dpp_u32<0x138>(old, v); }

// Segmented inclusive max-scan across a wavefront: segments are runs of equal
// key, keys ascending along the lanes.  Each lane gets the max of val over
// lanes [start of its run, lane].  Row shifts 1, 2, 4, 8 scan within rows of
// 16 lanes; the row broadcasts of lanes 15/47 and then 31 carry across rows.
__device__ __forceinline__ uint32_t seg_max_scan(uint32_t key, uint32_t val) {
#define ADACOMP_SEG_STEP(CTRL, ROWS)                                   \
    {                                                                   \
        const uint32_t k2 = dpp_u32<CTRL, ROWS>(kNoKey, key);          \
        const uint32_t v2 = dpp_u32<CTRL, ROWS>(0u, val);              \
        if (k2 == key) val = max(val, v2);                              \
    }
    ADACOMP_SEG_STEP(0x111, 0xf)
    ADACOMP_SEG_STEP(0x112, 0xf)
    ADACOMP_SEG_STEP(0x114, 0xf)
    ADACOMP_SEG_STEP(0x118, 0xf)
    ADACOMP_SEG_STEP(0x142, 0xa)
    ADACOMP_SEG_STEP(0x143, 0xc)
#undef ADACOMP_SEG_STEP
    return val;
}

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// One tile's inputs held in registers: residue and dW of VPT float4 per thread.
template <int VPT>
struct TileRegs {
    TileGeom tg;
    uint32_t tile;
    float rr[VPT][4];
    float dw[VPT][4];
};

// Issues the tile's loads without branches, so that the compiler can keep a
// prefetched tile in flight: every lane loads whole float4 (lanes past the
// tile reload its last float4).  Elements outside the tile are loaded but
// masked later; the flat buffers are padded to a multiple of 4 elements, so
// every float4 is inside them.
template <int THREADS, int VPT>
__device__ __forceinline__ void load_tile(TileRegs<VPT>& t, const SegDev* __restrict__ segs,
                                          const uint32_t* __restrict__ tile_seg,
                                          const uint32_t* __restrict__ vtiles, uint32_t it,
                                          const float* __restrict__ residue,
                                          const float* __restrict__ dW) {
    const int tid = threadIdx.x;
    t.tile = vtiles[it];
    const SegDev& sg = segs[tile_seg[t.tile]];
    t.tg = tile_geom(sg, sg.ct, t.tile);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const uint32_t vi = min(uint32_t(v * THREADS + tid), t.tg.nvec - 1u);
        const uint64_t e0 = t.tg.v0 + uint64_t(vi) * 4u;
        const f32x4 a = load4<ADACOMP_NT_R>(residue + e0);
        const f32x4 b = load4<ADACOMP_NT_DW>(dW + e0);
        t.rr[v][0] = a.x; t.rr[v][1] = a.y; t.rr[v][2] = a.z; t.rr[v][3] = a.w;
        t.dw[v][0] = b.x; t.dw[v][1] = b.y; t.dw[v][2] = b.z; t.dw[v][3] = b.w;
    }
}

// Everything a tile does after its inputs arrived.  lds: this tile's
// [2*bpt_max+1] words (bin maxima, then bin boundaries).
template <int THREADS, int VPT>
__device__ __forceinline__ void process_tile(const TileRegs<VPT>& in, uint32_t* lds,
                                             const SegDev* __restrict__ segs,
                                             const uint32_t* __restrict__ tile_seg,
                                             float* __restrict__ residue, uint8_t* __restrict__ msg,
                                             uint2* __restrict__ stage,
                                             uint32_t* __restrict__ tile_cnt,
                                             double* __restrict__ tile_gsum,
                                             float* __restrict__ bin_max_out,
                                             uint32_t* ch_tot) {
    constexpr int NW = THREADS / 64;
    constexpr int NCH = NW * VPT;   // wavefront chunks of 256 elements per tile
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const TileGeom& tg = in.tg;
    const SegDev sg = segs[tile_seg[in.tile]];
    const uint32_t lt = sg.lt, magic = sg.magic;
    uint32_t* smax = lds;                 // [bpt] bin maxima as float bits
    uint32_t* sbound = lds + sg.ct.bpt;      // [bpt + 1] survivors before each bin
    uint32_t* sfirst = sbound + sg.ct.bpt + 1;   // [bpt] LS only: first index of the maximum
    const bool ls = (sg.flags & ADACOMP_SEG_LS) != 0u;

    for (uint32_t b = tid; b < tg.nb; b += THREADS) {
        smax[b] = 0u;
        if (ls) sfirst[b] = kSentinel;
    }

    float g[VPT][4];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) g[v][c] = in.rr[v][c] + in.dw[v][c];   // G = residue + dW
    __syncthreads();   // smax cleared

    // ---- bin maxima: g_max(i) = max |G| over bin i ----
    if (lt >= 4u) {
        // A float4 then spans at most two bins: a head run and a tail run.
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int vi = v * THREADS + tid;
            const int x0 = vi * 4 - int(tg.lead);
            uint32_t hb = kSentinel, tb = kSentinel, mh = 0u, mt = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int x = x0 + c;
                if (vi < int(tg.nvec) && x >= 0 && x < int(tg.tlen)) {
                    const uint32_t b = div_bin(uint32_t(x), lt, magic);
                    const uint32_t m = __float_as_uint(fabsf(g[v][c]));
                    if (hb == kSentinel) { hb = b; tb = b; mh = m; mt = m; }
                    else if (b == hb) { mh = max(mh, m); mt = max(mt, m); }
                    else if (b == tb) { mt = max(mt, m); }
                    else { tb = b; mt = m; }
                }
            }
            const bool two = hb != tb;
            // The head run of a two-run lane continues the previous lane's
            // tail run: fold it there; otherwise the lane emits it itself.
            const uint32_t ptb = from_prev_lane(kNoKey, tb);
            if (two && ptb != hb) atomicMax(&smax[hb], mh);
            const uint32_t nhb = from_next_lane(kNoKey, two ? hb : kNoKey);
            const uint32_t nmh = from_next_lane(0u, mh);
            if (nhb == tb) mt = max(mt, nmh);
            const uint32_t val = seg_max_scan(tb, mt);
            const uint32_t nkey = from_next_lane(kNoKey, tb);
            if (nkey != tb && tb != kSentinel) atomicMax(&smax[tb], val);
        }
    } else {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int vi = v * THREADS + tid;
            const int x0 = vi * 4 - int(tg.lead);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int x = x0 + c;
                if (vi < int(tg.nvec) && x >= 0 && x < int(tg.tlen))
                    atomicMax(&smax[div_bin(uint32_t(x), lt, magic)],
                              __float_as_uint(fabsf(g[v][c])));
            }
        }
    }
    __syncthreads();

    if (ls) {
        // Hard local selection: the lowest index whose |G| is the (nonzero)
        // bin maximum.
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int vi = v * THREADS + tid;
            const int x0 = vi * 4 - int(tg.lead);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int x = x0 + c;
                if (vi < int(tg.nvec) && x >= 0 && x < int(tg.tlen)) {
                    const uint32_t b = div_bin(uint32_t(x), lt, magic);
                    const uint32_t m = __float_as_uint(fabsf(g[v][c]));
                    if (m != 0u && m == smax[b]) atomicMin(&sfirst[b], uint32_t(x));
                }
            }
        }
        __syncthreads();
    }

    // ---- selection: |H| >= g_max of the bin and G != 0 (LS: the first maximum) ----
    uint32_t sel[VPT];
    uint32_t wrank[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int vi = v * THREADS + tid;
        const int x0 = vi * 4 - int(tg.lead);
        uint32_t m = 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int x = x0 + c;
            if (vi < int(tg.nvec) && x >= 0 && x < int(tg.tlen)) {
                const uint32_t b = div_bin(uint32_t(x), lt, magic);
                const float gm = __uint_as_float(smax[b]);
                const float h = g[v][c] + in.dw[v][c];      // H = G + dW
                const bool take = ls ? sfirst[b] == uint32_t(x) : fabsf(h) >= gm && g[v][c] != 0.0f;
                if (take) m |= 1u << c;
            }
        }
        sel[v] = m;
        const uint64_t b0 = __ballot(m & 1u), b1 = __ballot(m & 2u);
        const uint64_t b2 = __ballot(m & 4u), b3 = __ballot(m & 8u);
        wrank[v] = mbcnt64(b0) + mbcnt64(b1) + mbcnt64(b2) + mbcnt64(b3);
        if (lane == 0) ch_tot[v * NW + wv] = __popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3);
    }
    __syncthreads();
    uint32_t total = 0;
    uint32_t cbase[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) cbase[v] = 0;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const uint32_t t = ch_tot[q];
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            if (q < v * NW + wv) cbase[v] += t;
        total += t;
    }

    // ---- survivors to staging, bin boundaries, residue <- G ----
    uint2* st = stage + tg.t0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int vi = v * THREADS + tid;
        const int x0 = vi * 4 - int(tg.lead);
        if (vi >= int(tg.nvec)) continue;
        uint32_t r = cbase[v] + wrank[v];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int x = x0 + c;
            if (x >= 0 && x < int(tg.tlen)) {
                const uint32_t b = div_bin(uint32_t(x), lt, magic);
                if (uint32_t(x) == b * lt) sbound[b] = r;
                if (sel[v] & (1u << c)) {
                    const uint32_t neg = g[v][c] < 0.0f ? 0x80000000u : 0u;
                    st[r] = make_uint2(neg | uint32_t(x), __float_as_uint(g[v][c]));
                    ++r;
                }
            }
        }
        const uint64_t e0 = tg.v0 + uint64_t(vi) * 4u;
        if (x0 >= 0 && x0 + 4 <= int(tg.tlen)) {
            f32x4 o;
            o.x = g[v][0]; o.y = g[v][1]; o.z = g[v][2]; o.w = g[v][3];
            store4<ADACOMP_NT_ST>(residue + e0, o);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int x = x0 + c;
                if (x >= 0 && x < int(tg.tlen)) residue[e0 + c] = g[v][c];
            }
        }
    }
    if (tid == 0) sbound[tg.nb] = total;
    __syncthreads();

    // ---- per-bin count words, optional g_max export, tile totals ----
    uint8_t* cw = msg + sg.count_off + uint64_t(tg.first_bin) * sg.wb;
    for (uint32_t b = tid; b < tg.nb; b += THREADS) {
        put_word(cw + uint64_t(b) * sg.wb, sg.wb, sbound[b + 1] - sbound[b]);
        if (bin_max_out) bin_max_out[sg.bin_base + tg.first_bin + b] = __uint_as_float(smax[b]);
    }
    if (wv == NW - 1) {
        // float64 sum of the tile's bin maxima in a fixed order
        double acc = 0.0;
        if (tg.nb <= 64) {
            if (lane == 0)
                for (uint32_t b = 0; b < tg.nb; ++b) acc += double(__uint_as_float(smax[b]));
        } else {
            for (uint32_t b = lane; b < tg.nb; b += 64) acc += double(__uint_as_float(smax[b]));
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d);
        }
        if (lane == 0) {
            tile_gsum[in.tile] = acc;
            tile_cnt[in.tile] = total;
        }
    }
}

// One workgroup per tile.
template <int THREADS, int VPT>
__global__ void __launch_bounds__(THREADS)
k_tile_pass(const SegDev* __restrict__ segs, const uint32_t* __restrict__ tile_seg,
            const uint32_t* __restrict__ vtiles, float* __restrict__ residue,
            const float* __restrict__ dW, uint8_t* __restrict__ msg, uint2* __restrict__ stage,
            uint32_t* __restrict__ tile_cnt, double* __restrict__ tile_gsum,
            float* __restrict__ bin_max_out) {
    constexpr int NCH = (THREADS / 64) * VPT;
    extern __shared__ uint32_t dyn[];
    __shared__ uint32_t ch_tot[NCH];
    TileRegs<VPT> a;
    load_tile<THREADS, VPT>(a, segs, tile_seg, vtiles, blockIdx.x, residue, dW);
    process_tile<THREADS, VPT>(a, dyn, segs, tile_seg, residue, msg, stage, tile_cnt, tile_gsum,
                               bin_max_out, ch_tot);
}

// Long bins (L_T > 4093): one workgroup per bin.  The bin is streamed twice
// in chunks of THREADS x VPT float4: the first pass finds g_max (and, for
// hard local selection, the first index holding it), the second forms G and
// H again, selects, compacts and writes the residue.  The second pass reads
// what the first one just brought on chip (non-temporal: it is the last use),
// so HBM traffic stays near 12 B/element while bins fit the caches (L_T =
// 5000: 40 KiB of residue and dW per workgroup) and only 2 float4 per array
// live in registers.
template <int THREADS, int VPT>
__global__ void __launch_bounds__(THREADS)
k_tile_pass_long(const SegDev* __restrict__ segs, const uint32_t* __restrict__ tile_seg,
                 const uint32_t* __restrict__ vtiles, float* __restrict__ residue,
                 const float* __restrict__ dW, uint8_t* __restrict__ msg, uint2* __restrict__ stage,
                 uint32_t* __restrict__ tile_cnt, double* __restrict__ tile_gsum,
                 float* __restrict__ bin_max_out) {
    constexpr int NW = THREADS / 64;
    constexpr int NCH = NW * VPT;
    constexpr uint32_t CV = THREADS * VPT;   // float4 per chunk
    __shared__ uint32_t red_m[NW], red_i[NW];
    __shared__ uint32_t ch_tot[NCH];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint32_t tile = vtiles[blockIdx.x];
    const SegDev sg = segs[tile_seg[tile]];
    const TileGeom tg = tile_geom(sg, sg.ct, tile);   // exactly one bin
    const bool ls = (sg.flags & ADACOMP_SEG_LS) != 0u;
    const int lead = int(tg.lead), tlen = int(tg.tlen);

    // ---- pass 1: g_max = max |G| over the bin, and its first index ----
    uint32_t m = 0u, mi = kSentinel;
    for (uint32_t c0 = 0; c0 < tg.nvec; c0 += CV) {
        f32x4 a[VPT], b[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t vi = min(c0 + uint32_t(v * THREADS + tid), tg.nvec - 1u);
            a[v] = load4<false>(residue + tg.v0 + uint64_t(vi) * 4u);
            b[v] = load4<false>(dW + tg.v0 + uint64_t(vi) * 4u);
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t vi = c0 + uint32_t(v * THREADS + tid);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int x = int(vi * 4) + c - lead;
                if (vi < tg.nvec && x >= 0 && x < tlen) {
                    const uint32_t mm = __float_as_uint(fabsf(a[v][c] + b[v][c]));
                    if (mm > m) { m = mm; mi = uint32_t(x); }   // x grows, so the first index is kept
                }
            }
        }
    }
    // largest |G|, ties to the lowest index
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t om = __shfl_xor(m, d), oi = __shfl_xor(mi, d);
        if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
    }
    if (lane == 0) { red_m[wv] = m; red_i[wv] = mi; }
    __syncthreads();
    m = red_m[0];
    mi = red_i[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        if (red_m[w] > m || (red_m[w] == m && red_i[w] < mi)) { m = red_m[w]; mi = red_i[w]; }
    const float gm = __uint_as_float(m);
    const uint32_t first = m != 0u ? mi : kSentinel;   // LS: nothing in an all-zero bin

    // ---- pass 2: selection, compaction to staging, residue <- G ----
#ifndef ADACOMP_LONG_NT2
#define ADACOMP_LONG_NT2 1
#endif
    uint32_t carry = 0;
    uint2* st = stage + tg.t0;
    for (uint32_t c0 = 0; c0 < tg.nvec; c0 += CV) {
        f32x4 a[VPT], b[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t vi = min(c0 + uint32_t(v * THREADS + tid), tg.nvec - 1u);
            a[v] = load4<ADACOMP_LONG_NT2>(residue + tg.v0 + uint64_t(vi) * 4u);
            b[v] = load4<ADACOMP_LONG_NT2>(dW + tg.v0 + uint64_t(vi) * 4u);
        }
        uint32_t sel[VPT], wrank[VPT];
        float g[VPT][4];
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t vi = c0 + uint32_t(v * THREADS + tid);
            uint32_t msk = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                g[v][c] = a[v][c] + b[v][c];                 // G = residue + dW
                const int x = int(vi * 4) + c - lead;
                if (vi < tg.nvec && x >= 0 && x < tlen) {
                    const float h = g[v][c] + b[v][c];      // H = G + dW
                    const bool take = ls ? uint32_t(x) == first : fabsf(h) >= gm && g[v][c] != 0.0f;
                    if (take) msk |= 1u << c;
                }
            }
            sel[v] = msk;
            const uint64_t b0 = __ballot(msk & 1u), b1 = __ballot(msk & 2u);
            const uint64_t b2 = __ballot(msk & 4u), b3 = __ballot(msk & 8u);
            wrank[v] = mbcnt64(b0) + mbcnt64(b1) + mbcnt64(b2) + mbcnt64(b3);
            if (lane == 0) ch_tot[v * NW + wv] = __popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3);
        }
        __syncthreads();
        uint32_t total = 0, cbase[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) cbase[v] = 0;
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            const uint32_t t = ch_tot[q];
#pragma unroll
            for (int v = 0; v < VPT; ++v)
                if (q < v * NW + wv) cbase[v] += t;
            total += t;
        }
        __syncthreads();   // ch_tot is rewritten by the next chunk
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t vi = c0 + uint32_t(v * THREADS + tid);
            if (vi >= tg.nvec) continue;
            const int x0 = int(vi * 4) - lead;
            uint32_t r = carry + cbase[v] + wrank[v];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (sel[v] & (1u << c)) {
                    const uint32_t neg = g[v][c] < 0.0f ? 0x80000000u : 0u;
                    st[r] = make_uint2(neg | uint32_t(x0 + c), __float_as_uint(g[v][c]));
                    ++r;
                }
            }
            const uint64_t e0 = tg.v0 + uint64_t(vi) * 4u;
            if (x0 >= 0 && x0 + 4 <= tlen) {
                f32x4 o;
                o.x = g[v][0]; o.y = g[v][1]; o.z = g[v][2]; o.w = g[v][3];
                store4<ADACOMP_NT_ST>(residue + e0, o);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int x = x0 + c;
                    if (x >= 0 && x < tlen) residue[e0 + c] = g[v][c];
                }
            }
        }
        carry += total;
    }
    if (tid == 0) {
        put_word(msg + sg.count_off + uint64_t(tg.first_bin) * sg.wb, sg.wb, carry);
        if (bin_max_out) bin_max_out[sg.bin_base + tg.first_bin] = gm;
        tile_gsum[tile] = double(gm);
        tile_cnt[tile] = carry;
    }
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one value per thread (256 threads).
// ---------------------------------------------------------------------------
template <int THREADS>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds_w,
                                                         uint32_t* total) {
    constexpr int NW = THREADS / 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = __shfl_up(inc, d);
        if (lane >= d) inc += t;
    }
    if (lane == 63) lds_w[wv] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = lds_w[w];
        if (w < wv) before += x;
        all += x;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// Chunk scan: tiles [chunk_tile_begin[c], chunk_tile_begin[c+1]) <= 1024.
__global__ void __launch_bounds__(256)
k_chunk_scan(const uint32_t* __restrict__ chunk_tile_begin, const uint32_t* __restrict__ tile_cnt,
             const double* __restrict__ tile_gsum, uint32_t* __restrict__ tile_off,
             uint32_t* __restrict__ chunk_cnt, double* __restrict__ chunk_gsum) {
    __shared__ uint32_t lw[4];
    __shared__ double lg[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint32_t c = blockIdx.x;
    const uint32_t tb = chunk_tile_begin[c], n = chunk_tile_begin[c + 1] - tb;
    uint32_t cnt[4];
    uint32_t mine = 0;
    double gs = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = uint32_t(tid) * 4u + i;
        cnt[i] = t < n ? tile_cnt[tb + t] : 0u;
        if (t < n) gs += tile_gsum[tb + t];
        mine += cnt[i];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<256>(mine, lw, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = uint32_t(tid) * 4u + i;
        if (t < n) tile_off[tb + t] = run;
        run += cnt[i];
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) gs += __shfl_xor(gs, d);
    if (lane == 0) lg[wv] = gs;
    __syncthreads();
    if (tid == 0) {
        chunk_cnt[c] = total;
        chunk_gsum[c] = ((lg[0] + lg[1]) + lg[2]) + lg[3];
    }
}

// Finalize: one block of 256 threads.
__global__ void __launch_bounds__(256)
k_finalize(const SegDev* __restrict__ segs, uint32_t nseg, uint32_t plan_hash,
           uint64_t entries_begin, const uint32_t* __restrict__ chunk_cnt,
           const double* __restrict__ chunk_gsum, uint32_t* __restrict__ chunk_base,
           float* __restrict__ seg_s, uint32_t* __restrict__ seg_nsurv,
           uint64_t* __restrict__ seg_eoff, uint64_t* __restrict__ seg_sbase,
           uint8_t* __restrict__ msg) {
    __shared__ uint64_t lsz[4], lns[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // s and survivor totals per segment; chunk bases within the segment.
    for (uint32_t l = tid; l < nseg; l += 256) {
        const SegDev sg = segs[l];
        double acc = 0.0;
        uint32_t run = 0;
        for (uint32_t c = 0; c < sg.ct.nchunks; ++c) {
            const uint32_t ci = sg.ct.chunk_begin + c;
            acc += chunk_gsum[ci];
            chunk_base[ci] = run;
            run += chunk_cnt[ci];
        }
        // s = mean of the bin maxima, rounded once to float32.
        seg_s[l] = float(acc / double(sg.nbins));
        seg_nsurv[l] = run;
        // Zero the padding after the count region.
        const uint64_t cend = sg.count_off + uint64_t(sg.nbins) * sg.wb;
        for (uint64_t p = cend; p < rup16(cend); ++p) msg[p] = 0;
    }
    __syncthreads();
    // Entry regions in table order, each 16-byte aligned, and the number of
    // survivors before each segment.
    uint64_t carry = 0, surv = 0;
    for (uint32_t base = 0; base < nseg; base += 256) {
        const uint32_t l = base + tid;
        uint64_t sz = 0, ns = 0;
        if (l < nseg) {
            ns = seg_nsurv[l];
            sz = rup16(ns * segs[l].wb);
        }
        uint64_t isz = sz, ins = ns;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint64_t t = __shfl_up(isz, d);
            const uint64_t t2 = __shfl_up(ins, d);
            if (lane >= d) { isz += t; ins += t2; }
        }
        if (lane == 63) { lsz[wv] = isz; lns[wv] = ins; }
        __syncthreads();
        uint64_t bsz = 0, bns = 0, asz = 0, ans = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < wv) { bsz += lsz[w]; bns += lns[w]; }
            asz += lsz[w];
            ans += lns[w];
        }
        __syncthreads();
        if (l < nseg) {
            const uint64_t eoff = entries_begin + carry + bsz + isz - sz;
            seg_eoff[l] = eoff;
            seg_sbase[l] = surv + bns + ins - ns;
            uint8_t* d = msg + 32 + 16 * uint64_t(l);
            *reinterpret_cast<float*>(d) = seg_s[l];
            *reinterpret_cast<uint32_t*>(d + 4) = uint32_t(ns);
            *reinterpret_cast<uint64_t*>(d + 8) = eoff;
            const uint64_t wend = eoff + ns * segs[l].wb;
            for (uint64_t p = wend; p < eoff + sz; ++p) msg[p] = 0;
        }
        carry += asz;
        surv += ans;
    }
    if (tid == 0) {
        *reinterpret_cast<uint32_t*>(msg) = 0x43414441u;
        *reinterpret_cast<uint16_t*>(msg + 4) = 1;
        *reinterpret_cast<uint16_t*>(msg + 6) = 0;
        *reinterpret_cast<uint32_t*>(msg + 8) = nseg;
        *reinterpret_cast<uint32_t*>(msg + 12) = plan_hash;
        *reinterpret_cast<uint64_t*>(msg + 16) = entries_begin + carry;
        *reinterpret_cast<uint64_t*>(msg + 24) = surv;
        seg_sbase[nseg] = surv;
    }
}

// Encode + residue fix-up, balanced over survivors.  The survivors of the
// table are numbered in message order (segment, bin, in-bin index);
// wavefront w of W takes survivors [S*w/W, S*(w+1)/W).  It finds the tile
// holding its first survivor with three 64-way searches (segment, scan chunk,
// tile), then walks the tiles from there 64 at a time: lane i holds tile i's
// metadata, a wavefront scan of the survivor counts flattens their
// survivors, and the lanes take them 64 at a time, with the staged pairs of
// kEncBatch rounds loaded before any of them is used.  Only wavefront-level
// operations are used, so every wavefront ends on its own.
#ifndef ADACOMP_ENC_BATCH
#define ADACOMP_ENC_BATCH 8
#endif
constexpr int kEncBatch = ADACOMP_ENC_BATCH;
constexpr uint32_t kEncMaxBlocks = 2048;   // 8192 wavefronts: one per wavefront slot of the chip

// Largest i in [0, n) with key(i) <= x, for key nondecreasing with
// key(0) = 0 <= x; wavefront-uniform, and *kv = key(i).  Each round probes
// 64 evenly spaced keys; the last round probes the answer itself.
template <class Key>
__device__ __forceinline__ uint32_t wave_last_le(uint32_t n, uint64_t x, Key key, uint64_t* kv) {
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t lo = 0, len = n;
    uint64_t v = 0;
    while (len > 1) {
        const uint32_t step = (len + 63u) / 64u;
        const uint32_t off = lane * step;
        const uint64_t k = off < len ? key(lo + off) : ~uint64_t(0);
        const uint64_t m = __ballot(k <= x);     // a prefix of the lanes, lane 0 included
        const uint32_t j = 63u - uint32_t(__clzll(m));
        v = (uint64_t(__shfl(uint32_t(k >> 32), int(j))) << 32) | __shfl(uint32_t(k), int(j));
        lo += j * step;
        len = min(step, len - j * step);
    }
    *kv = v;
    return lo;
}

__global__ void __launch_bounds__(256)
k_encode(const SegDev* __restrict__ segs, uint32_t nseg, const uint32_t* __restrict__ tile_seg,
         const uint2* __restrict__ stage, const uint32_t* __restrict__ tile_cnt,
         const uint32_t* __restrict__ tile_off, const uint32_t* __restrict__ chunk_base,
         const float* __restrict__ seg_s, const uint64_t* __restrict__ seg_eoff,
         const uint64_t* __restrict__ seg_sbase, uint8_t* __restrict__ msg,
         float* __restrict__ residue, uint32_t ntiles) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t W = gridDim.x * 4u, w = blockIdx.x * 4u + (threadIdx.x >> 6);
    const uint64_t S = seg_sbase[nseg];
    const uint64_t a = S * w / W, b = S * (w + 1) / W;
    if (a >= b) return;   // wavefront-uniform

    // The tile holding survivor a, and a's rank in it.
    uint64_t kv;
    const uint32_t l = wave_last_le(nseg, a, [&](uint32_t i) { return seg_sbase[i]; }, &kv);
    const SegDev sg = segs[l];
    const uint64_t ra = a - kv;
    const uint32_t c = wave_last_le(sg.ct.nchunks, ra, [&](uint32_t i) {
        return uint64_t(chunk_base[sg.ct.chunk_begin + i]);
    }, &kv);
    const uint64_t rc = ra - kv;
    const uint32_t tb = sg.ct.tile_begin + c * kChunkTiles;
    const uint32_t nt = min(kChunkTiles, sg.ct.ntiles - c * kChunkTiles);
    const uint32_t t = wave_last_le(nt, rc, [&](uint32_t i) { return uint64_t(tile_off[tb + i]); }, &kv);
    uint32_t r0 = uint32_t(rc - kv);
    uint32_t tile0 = tb + t;
    uint64_t remaining = b - a;

    while (remaining > 0 && tile0 < ntiles) {   // the tile bound only guards against bad counts
        const uint32_t tl = tile0 + lane;
        uint32_t cnt = 0, si = 0;
        if (tl < ntiles) {
            cnt = tile_cnt[tl];
            si = tile_seg[tl];
        }
        const uint32_t skip = lane == 0 ? r0 : 0u;   // survivors of the first tile already taken
        cnt -= skip;
        uint32_t incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t v = __shfl_up(incl, d);
            if (lane >= uint32_t(d)) incl += v;
        }
        const uint32_t total = __shfl(incl, 63);
        const uint32_t take = uint32_t(min<uint64_t>(total, remaining));
        const uint32_t excl = incl - cnt;
        // This lane's tile: flat index of its first element, message byte of
        // its first word taken here, s, L_T | word bytes, magic.
        uint64_t t0 = 0, eat = 0;
        float s = 0.0f;
        uint32_t ltwb = 0, mag = 0;
        if (cnt != 0 && excl < take) {
            const SegDev q = segs[si];
            const TileGeom tg = tile_geom(q, q.ct, tl);
            const uint32_t chunk = q.ct.chunk_begin + (tl - q.ct.tile_begin) / kChunkTiles;
            const uint64_t rank = uint64_t(chunk_base[chunk]) + tile_off[tl] + skip;
            t0 = tg.t0;
            eat = seg_eoff[si] + rank * q.wb;
            s = seg_s[si];
            ltwb = (q.lt << 2) | q.wb;
            mag = q.magic;
        }
        for (uint32_t base = 0; base < take; base += 64u * kEncBatch) {   // wavefront-uniform
            uint32_t own[kEncBatch], k[kEncBatch];
            uint64_t tt[kEncBatch];
            uint2 p[kEncBatch];
            // Owners and staged pairs first; lanes past the end reload the last survivor.
#pragma unroll
            for (int u = 0; u < kEncBatch; ++u) {
                const uint32_t e = min(base + 64u * u + lane, take - 1u);
                uint32_t L = 0;   // lanes whose survivors all precede e
#pragma unroll
                for (uint32_t bit = 32; bit >= 1; bit >>= 1)
                    if (__shfl(incl, int(L + bit - 1u)) <= e) L += bit;
                own[u] = L;
                k[u] = e - __shfl(excl, int(L));
                tt[u] = (uint64_t(__shfl(uint32_t(t0 >> 32), int(L))) << 32) |
                        __shfl(uint32_t(t0), int(L));
                p[u] = stage[tt[u] + (L == 0 ? r0 : 0u) + k[u]];
            }
#pragma unroll
            for (int u = 0; u < kEncBatch; ++u) {
                const uint32_t L = own[u];
                const uint64_t ea = (uint64_t(__shfl(uint32_t(eat >> 32), int(L))) << 32) |
                                    __shfl(uint32_t(eat), int(L));
                const uint32_t lw = __shfl(ltwb, int(L)), mg = __shfl(mag, int(L));
                const float sv = __shfl(s, int(L));
                if (base + 64u * u + lane < take) {
                    const uint32_t lt = lw >> 2, wb = lw & 3u;
                    const uint32_t x = p[u].x & 0x7FFFFFFFu;
                    const uint32_t neg = p[u].x >> 31;
                    const uint32_t bin = div_bin(x, lt, mg);
                    const uint32_t topbit = wb == 1u ? 7u : 15u;
                    put_word(msg + ea + uint64_t(k[u]) * wb, wb, (neg << topbit) | (x - bin * lt));
                    const float gv = __uint_as_float(p[u].y);
                    // residue <- G - G_q with G_q = sign(G) * s
                    residue[tt[u] + x] = neg ? gv + sv : gv - sv;
                }
            }
        }
        remaining -= take;
        tile0 += 64u;
        r0 = 0;
    }
}

// ---------------------------------------------------------------------------
// Decode-accumulate, over decode tiles (TileSpec dt of each layer).
// ---------------------------------------------------------------------------
struct MsgPtrs {
    const uint8_t* p[ADACOMP_MAX_MESSAGES];
};

struct DecodeWs {
    uint32_t* status;     // [1]
    uint32_t* dcnt;       // [K*DT]
    uint32_t* doff;       // [K*DT]
    uint32_t* dchunk_cnt; // [K*DC]
    uint32_t* dchunk_base;// [K*DC]
    float* dseg_s;        // [K*nseg]
    uint64_t* dseg_eoff;  // [K*nseg]
    uint32_t* dvalid;     // [K]
};

__device__ __forceinline__ bool header_matches(const uint8_t* m, uint32_t nseg, uint32_t plan_hash) {
    return *reinterpret_cast<const uint32_t*>(m) == 0x43414441u &&
           *reinterpret_cast<const uint16_t*>(m + 4) == 1 &&
           *reinterpret_cast<const uint32_t*>(m + 8) == nseg &&
           *reinterpret_cast<const uint32_t*>(m + 12) == plan_hash;
}

// Sum of the count words in message bytes [a0, a1), read as the aligned
// 32-bit words that cover them (count regions start 16-byte aligned and are
// zero-padded to 16 bytes, so those words lie inside the message).
__device__ __forceinline__ uint32_t sum_count_words(const uint8_t* m, uint64_t a0, uint64_t a1,
                                                    uint32_t wb) {
    typedef const __attribute__((address_space(1))) uint32_t* gu32;
    uint32_t s = 0;
#pragma unroll 4
    for (uint64_t d = a0 & ~uint64_t(3); d < a1; d += 4) {
        uint32_t v = *(gu32)(m + d);
        if (d < a0) v &= ~0u << (8u * uint32_t(a0 - d));          // bytes before a0
        if (d + 4 > a1) v &= ~0u >> (8u * uint32_t(d + 4 - a1));  // bytes from a1 on
        s += wb == 1u ? (v & 0xFFu) + ((v >> 8) & 0xFFu) + ((v >> 16) & 0xFFu) + (v >> 24)
                      : (v & 0xFFFFu) + (v >> 16);
    }
    return s;
}

// Per (chunk of decode tiles, message): survivors of each decode tile from
// the count words, offsets within the chunk, chunk totals.
__global__ void __launch_bounds__(256)
k_decode_count(MsgPtrs msgs, const SegDev* __restrict__ segs,
               const uint32_t* __restrict__ chunk_tile_begin, const uint32_t* __restrict__ chunk_seg,
               uint32_t DT, uint32_t DC, uint32_t nseg, uint32_t plan_hash, DecodeWs ws) {
    __shared__ uint32_t lw[4];
    const uint32_t c = blockIdx.x, k = blockIdx.y;
    const uint8_t* m = msgs.p[k];
    // A message made for another table is never read past its header.
    const bool ok = header_matches(m, nseg, plan_hash);
    const SegDev sg = segs[chunk_seg[c]];
    const uint32_t tb = chunk_tile_begin[c], n = chunk_tile_begin[c + 1] - tb;
    uint32_t cnt[4];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = threadIdx.x * 4u + i;
        uint32_t s = 0;
        if (ok && t < n) {
            const uint32_t first_bin = (tb + t - sg.dt.tile_begin) * sg.dt.bpt;
            const uint32_t nb = min(sg.dt.bpt, sg.nbins - first_bin);
            const uint64_t a0 = sg.count_off + uint64_t(first_bin) * sg.wb;
            s = sum_count_words(m, a0, a0 + uint64_t(nb) * sg.wb, sg.wb);
        }
        cnt[i] = s;
        mine += s;
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<256>(mine, lw, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = threadIdx.x * 4u + i;
        if (t < n) {
            ws.dcnt[uint64_t(k) * DT + tb + t] = cnt[i];
            ws.doff[uint64_t(k) * DT + tb + t] = run;
        }
        run += cnt[i];
    }
    if (threadIdx.x == 0) ws.dchunk_cnt[uint64_t(k) * DC + c] = total;
}

// One block: message validity, per-segment s and entry offsets, chunk bases.
__global__ void __launch_bounds__(256)
k_decode_base(MsgPtrs msgs, uint32_t K, const SegDev* __restrict__ segs, uint32_t nseg,
              uint32_t plan_hash, uint32_t DC, DecodeWs ws) {
    __shared__ uint32_t valid[ADACOMP_MAX_MESSAGES];
    __shared__ uint32_t bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    for (uint32_t k = threadIdx.x; k < K; k += 256) {
        const bool ok = header_matches(msgs.p[k], nseg, plan_hash);
        valid[k] = ok ? 1u : 0u;
        ws.dvalid[k] = ok ? 1u : 0u;
        if (!ok) atomicAdd(&bad, 1u);
    }
    __syncthreads();
    for (uint64_t i = threadIdx.x; i < uint64_t(K) * nseg; i += 256) {
        const uint32_t k = uint32_t(i / nseg), l = uint32_t(i % nseg);
        float s = 0.0f;
        uint64_t eoff = 0;
        if (valid[k]) {
            const uint8_t* d = msgs.p[k] + 32 + 16 * uint64_t(l);
            s = *reinterpret_cast<const float*>(d);
            eoff = *reinterpret_cast<const uint64_t*>(d + 8);
        }
        ws.dseg_s[i] = s;
        ws.dseg_eoff[i] = eoff;
        const SegDev sg = segs[l];
        uint32_t run = 0;
        for (uint32_t c = 0; c < sg.dt.nchunks; ++c) {
            const uint64_t ci = uint64_t(k) * DC + sg.dt.chunk_begin + c;
            ws.dchunk_base[ci] = run;
            run += ws.dchunk_cnt[ci];
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) *ws.status = bad;
}

// Index word at byte address a (w = 8 or 16 bits), read as the aligned
// 16-bit word that contains it; messages are 16-byte aligned and padded to a
// multiple of 16 bytes, so the read stays inside the message.
// The address is formed from integers kept in LDS, so it is cast to a
// global-address-space pointer (a global load, not a flat one).
typedef const __attribute__((address_space(1))) uint16_t* global_u16_ptr;

#ifndef ADACOMP_DEC_BATCH
#define ADACOMP_DEC_BATCH 2
#endif
constexpr int kDecBatch = ADACOMP_DEC_BATCH;   // entry rounds whose loads are issued together

__device__ __forceinline__ uint32_t word_at(uint64_t a, uint32_t wb) {
    const uint32_t w16 = *(global_u16_ptr)(a & ~uint64_t(1));
    return wb == 1u ? (w16 >> (8u * uint32_t(a & 1u))) & 0xFFu : w16;
}

// Per decode tile: out[j] = (accumulate ? out[j] : +0) + q_0[j] + q_1[j] + ...
// in message order, only at transmitted j.  LDS_ACC keeps the tile in LDS;
// otherwise (bins longer than 4093) the tile is accumulated in place in out.
// Messages are taken in groups of KG (KG <= 64; their bin prefixes fill the
// LDS words given at launch).  The tile's bins are split between the
// wavefronts; each wavefront gathers the entries of its bins for the whole
// group (message-major) 64 at a time and adds them message by message.  One
// wavefront's LDS operations execute in program order, so the additions to
// an element happen in message order without block barriers.
// Dynamic LDS: [acc_words floats if LDS_ACC][KG u64 entry addresses][K
// floats s][NW*(KG+1) u32 per-wavefront flat prefixes][KG*pstride u32 bin
// prefixes].  Everything else about the tile comes from its descriptor.

template <int THREADS, bool LDS_ACC>
__global__ void __launch_bounds__(THREADS)
k_decode_apply(MsgPtrs msgs, uint32_t K, uint32_t KG, uint32_t pstride,
               const DecDesc* __restrict__ descs, uint32_t DT, uint32_t DC, uint32_t nseg,
               DecodeWs ws, float* __restrict__ out, int accumulate, uint32_t acc_words) {
    constexpr int NW = THREADS / 64;
    extern __shared__ uint64_t dyn64[];
    uint32_t* dyn = reinterpret_cast<uint32_t*>(dyn64);
    const uint32_t accw = LDS_ACC ? (acc_words + 1u) & ~1u : 0u;   // keep 8-byte alignment
    uint64_t* eaddr = reinterpret_cast<uint64_t*>(dyn + accw);
    float* ks = reinterpret_cast<float*>(eaddr + KG);
    uint32_t* wfk_all = reinterpret_cast<uint32_t*>(ks + K);   // [NW][KG + 1]
    uint32_t* pref = wfk_all + NW * (KG + 1);             // [KG][pstride]

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const DecDesc dd = descs[blockIdx.x];
    const uint64_t v0 = dd.t0 & ~uint64_t(3);
    const uint32_t lead = uint32_t(dd.t0 - v0);
    const uint32_t nvec = (lead + dd.tlen + 3u) >> 2;
    const uint32_t nb = dd.nb, tlen = dd.tlen;
    float* acc = LDS_ACC ? reinterpret_cast<float*>(dyn) : out + v0;
    const uint32_t wb = dd.wb, lt = dd.lt;
    const uint32_t topbit = wb == 1u ? 7u : 15u;
    const uint32_t wb0 = nb * uint32_t(wv) / NW, wb1 = nb * uint32_t(wv + 1) / NW;
    uint32_t* wfk = wfk_all + wv * (KG + 1);

    for (uint32_t k = tid; k < K; k += THREADS) ks[k] = ws.dseg_s[uint64_t(k) * nseg + dd.si];
    // Initial values: +0, or out.
    for (uint32_t vi = tid; vi < nvec; vi += THREADS) {
        const int x0 = int(vi * 4) - int(lead);
        const uint64_t e0 = v0 + uint64_t(vi) * 4u;
        if (x0 >= 0 && x0 + 4 <= int(tlen)) {
            if (LDS_ACC) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                if (accumulate) a = load4<true>(out + e0);
                *reinterpret_cast<f32x4*>(acc + vi * 4) = a;
            } else if (!accumulate) {
                store4<false>(out + e0, f32x4{0.f, 0.f, 0.f, 0.f});
            }
        } else {
            for (int c = 0; c < 4; ++c) {
                const int x = x0 + c;
                if (x >= 0 && x < int(tlen)) {
                    if (LDS_ACC) acc[vi * 4 + c] = accumulate ? out[e0 + c] : 0.0f;
                    else if (!accumulate) out[e0 + c] = 0.0f;
                }
            }
        }
    }

    for (uint32_t k0 = 0; k0 < K; k0 += KG) {
        const uint32_t kn = min(KG, K - k0);
        __syncthreads();   // bases staged; the previous group is done with pref
        // Count words of the tile's bins for this group of messages (the
        // message pointer and validity are read directly, not from LDS, so
        // these loads wait only for the descriptor).
        for (uint32_t i = tid; i < kn * nb; i += THREADS) {
            const uint32_t kk = i / nb, b = i - kk * nb;
            const uint32_t k = k0 + kk;
            uint32_t cw = 0;
            if (ws.dvalid[k])
                cw = word_at(reinterpret_cast<uint64_t>(msgs.p[k]) + dd.count_at + uint64_t(b) * wb, wb);
            pref[kk * pstride + b + 1] = cw;
        }
        if (tid < int(kn)) {
            const uint32_t k = k0 + tid;
            const uint64_t base = uint64_t(ws.dchunk_base[uint64_t(k) * DC + dd.chunk]) +
                                  ws.doff[uint64_t(k) * DT + dd.tile];
            eaddr[tid] = reinterpret_cast<uint64_t>(msgs.p[k]) +
                         ws.dseg_eoff[uint64_t(k) * nseg + dd.si] + base * wb;
        }
        __syncthreads();
        // Per-message exclusive prefix over the tile's bins.
        if (nb <= 32) {
            if (tid < int(kn)) {   // one thread per message
                uint32_t* pr = pref + tid * pstride;
                uint32_t run = 0;
                pr[0] = 0;
                for (uint32_t b = 0; b < nb; ++b) {
                    run += pr[b + 1];
                    pr[b + 1] = run;
                }
            }
        } else {
            for (uint32_t kk = wv; kk < kn; kk += NW) {   // one wavefront per message
                uint32_t* pr = pref + kk * pstride;
                uint32_t carry = 0;
                for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
                    const uint32_t b = b0 + lane;
                    const uint32_t v = b < nb ? pr[b + 1] : 0u;
                    uint32_t inc = v;
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const uint32_t t = __shfl_up(inc, d);
                        if (lane >= d) inc += t;
                    }
                    if (b < nb) pr[b + 1] = carry + inc;
                    carry += __shfl(inc, 63);
                }
                if (lane == 0) pr[0] = 0;
            }
        }
        __syncthreads();
        if (wb0 >= wb1) continue;   // no bins for this wavefront
        // This wavefront's entries, message-major: lane kk holds message kk's
        // count over the wavefront's bins; wfk is their exclusive prefix.
        {
            const uint32_t c = uint32_t(lane) < kn
                                   ? pref[lane * pstride + wb1] - pref[lane * pstride + wb0]
                                   : 0u;
            uint32_t inc = c;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t t = __shfl_up(inc, d);
                if (lane >= d) inc += t;
            }
            if (uint32_t(lane) < kn) wfk[lane + 1] = inc;
            if (lane == 0) wfk[0] = 0;
        }
        const uint32_t Ew = wfk[kn];
        // kDecBatch rounds of 64 entries: every entry word of the batch is
        // requested before any is used, then the rounds are applied in order.
        for (uint32_t i0 = 0; i0 < Ew; i0 += 64u * kDecBatch) {
            uint32_t kof[kDecBatch], xs[kDecBatch], words[kDecBatch];
#pragma unroll
            for (int u = 0; u < kDecBatch; ++u) {
                const uint32_t ii = min(i0 + 64u * u + uint32_t(lane), Ew - 1u);
                uint32_t lo = 0, hi = kn;   // wfk[lo] <= ii < wfk[hi]
                while (hi - lo > 1) {
                    const uint32_t mid = (lo + hi) >> 1;
                    if (wfk[mid] <= ii) lo = mid; else hi = mid;
                }
                const uint32_t* pr = pref + lo * pstride;
                const uint32_t e = ii - wfk[lo] + pr[wb0];
                uint32_t bl = wb0, bh = wb1;   // pr[bl] <= e < pr[bh]
                while (bh - bl > 1) {
                    const uint32_t mid = (bl + bh) >> 1;
                    if (pr[mid] <= e) bl = mid; else bh = mid;
                }
                kof[u] = lo;
                xs[u] = bl * lt;
                words[u] = word_at(eaddr[lo] + uint64_t(e) * wb, wb);
            }
#pragma unroll
            for (int u = 0; u < kDecBatch; ++u) {
                const uint32_t r0 = i0 + 64u * u;
                if (r0 >= Ew) break;   // wavefront-uniform
                const uint32_t lo = kof[u];
                const uint32_t word = words[u];
                const uint32_t idx = word & ((1u << topbit) - 1u);
                const uint32_t x = xs[u] + idx;
                const float sk = ks[k0 + lo];
                const float q = (word >> topbit) ? -sk : sk;
                const bool apply = r0 + uint32_t(lane) < Ew && idx < lt && x < tlen;
                // Messages present in this round, applied in order.
                const uint32_t klo = __builtin_amdgcn_readfirstlane(lo);
                const uint32_t khi = __shfl(lo, int(min(Ew - r0, 64u) - 1u));
                for (uint32_t kk = klo; kk <= khi; ++kk) {
                    if (apply && lo == kk) acc[x + lead] = acc[x + lead] + q;
                    if (!LDS_ACC) __threadfence_block();
                }
            }
        }
    }
    if (LDS_ACC) {
        __syncthreads();
        for (uint32_t vi = tid; vi < nvec; vi += THREADS) {
            const int x0 = int(vi * 4) - int(lead);
            const uint64_t e0 = v0 + uint64_t(vi) * 4u;
            if (x0 >= 0 && x0 + 4 <= int(tlen)) {
                store4<true>(out + e0, *reinterpret_cast<const f32x4*>(acc + vi * 4));
            } else {
                for (int c = 0; c < 4; ++c) {
                    const int x = x0 + c;
                    if (x >= 0 && x < int(tlen)) out[e0 + c] = acc[vi * 4 + c];
                }
            }
        }
    }
}

}  // namespace adacomp
