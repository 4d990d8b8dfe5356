// Compress, dense tile pass (and the long-bin variant) for gfx950.
//
// Method: "AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
// page, definition paragraph and Mechanism claim on local-bin soft threshold
// and mean-g_max quantization (Algorithm 2); word widths from its Application
// claim (Table 2).
#pragma once

#include "common.hpp"

namespace adacomp {

// ---------------------------------------------------------------------------
// Compress, dense tile pass.
// ---------------------------------------------------------------------------
constexpr uint32_t kNoKey = 0xFFFFFFFEu;   // never a bin index nor kSentinel

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
        const f32x4 a = load4<kNtLoadResidue>(residue + e0);
        const f32x4 b = load4<kNtLoadDw>(dW + e0);
        t.rr[v][0] = a.x; t.rr[v][1] = a.y; t.rr[v][2] = a.z; t.rr[v][3] = a.w;
        t.dw[v][0] = b.x; t.dw[v][1] = b.y; t.dw[v][2] = b.z; t.dw[v][3] = b.w;
    }
}

// Everything a tile does after its inputs arrived.  lds: this tile's
// 2 * bpt_max + 1 words (bin maxima, then bin boundaries), followed, when
// the plan has hard local selection layers, by bpt_max words for each
// bin's first maximum.
template <int THREADS, int VPT, bool NTS>
__device__ __forceinline__ void process_tile(const TileRegs<VPT>& in, uint32_t* lds,
                                             const SegDev* __restrict__ segs,
                                             const uint32_t* __restrict__ tile_seg,
                                             float* __restrict__ residue, uint8_t* __restrict__ msg,
                                             uint32_t* __restrict__ stage,
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

    // Per element, computed once for every pass below: G, its bin within
    // the tile, whether it lies in the tile (bit c of vm[v]) and whether it
    // starts its bin (bit c of fb[v]).
    float g[VPT][4];
    uint32_t bn[VPT][4];
    uint32_t vm[VPT], fb[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int vi = v * THREADS + tid;
        const int x0 = vi * 4 - int(tg.lead);
        uint32_t prev = x0 > 0 ? div_bin(uint32_t(x0 - 1), lt, magic) : ~0u;   // bin of x0 - 1
        vm[v] = 0u;
        fb[v] = 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int x = x0 + c;
            g[v][c] = in.rr[v][c] + in.dw[v][c];   // G = residue + dW
            bn[v][c] = div_bin(uint32_t(max(x, 0)), lt, magic);
            if (vi < int(tg.nvec) && x >= 0 && x < int(tg.tlen)) vm[v] |= 1u << c;
            if (x == 0 || (x > 0 && bn[v][c] != prev)) fb[v] |= 1u << c;   // a bin starts at x
            prev = bn[v][c];
        }
    }
    __syncthreads();   // smax cleared

    // ---- bin maxima: g_max(i) = max |G| over bin i ----
    if (lt >= 4u) {
        // A float4 then spans at most two bins: a head run and a tail run.
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            // Head run: the bin of the first element in the tile; tail run:
            // the bin of the last (a float4 spans at most two bins; elements
            // before the tile have bin 0, the first element's, and elements
            // past it are clamped to the tile's last bin, the last element's).
            // Maxima without branches; no element in the tile: no runs.
            const uint32_t valid = vm[v];
            const uint32_t hb = valid != 0u ? bn[v][0] : kSentinel;
            const uint32_t tb = valid != 0u ? min(bn[v][3], tg.nb - 1u) : kSentinel;
            uint32_t mh = 0u, mt = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t m = ((valid >> c) & 1u) ? __float_as_uint(fabsf(g[v][c])) : 0u;
                mh = max(mh, bn[v][c] == hb ? m : 0u);
                mt = max(mt, bn[v][c] == tb ? m : 0u);
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
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if ((vm[v] >> c) & 1u)
                    atomicMax(&smax[bn[v][c]], __float_as_uint(fabsf(g[v][c])));
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
                if ((vm[v] >> c) & 1u) {
                    const uint32_t b = bn[v][c];
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
            if ((vm[v] >> c) & 1u) {
                const uint32_t b = bn[v][c];
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
    // Survivor r's key at st[r]; when the tile's region holds both, its G at
    // st[total + r] as well, so that the finish can read it with the key.
    uint32_t* st = stage + tg.t0;
    const bool pair = 2u * total <= tg.tlen;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int vi = v * THREADS + tid;
        const int x0 = vi * 4 - int(tg.lead);
        if (vi >= int(tg.nvec)) continue;
        uint32_t r = cbase[v] + wrank[v];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int x = x0 + c;
            if ((vm[v] >> c) & 1u) {
                const uint32_t b = bn[v][c];
                if ((fb[v] >> c) & 1u) sbound[b] = r;
                if (sel[v] & (1u << c)) {
                    st[r] = (g[v][c] < 0.0f ? 0x80000000u : 0u) | uint32_t(x);
                    if (pair) st[total + r] = __float_as_uint(g[v][c]);
                    ++r;
                }
            }
        }
        const uint64_t e0 = tg.v0 + uint64_t(vi) * 4u;
        if (vm[v] == 15u) {
            f32x4 o;
            o.x = g[v][0]; o.y = g[v][1]; o.z = g[v][2]; o.w = g[v][3];
            store4<NTS>(residue + e0, o);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if ((vm[v] >> c) & 1u) residue[e0 + c] = g[v][c];
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

// One workgroup per tile.  NTS: non-temporal residue stores.
template <int THREADS, int VPT, bool NTS>
__global__ void __launch_bounds__(THREADS)
k_tile_pass(const SegDev* __restrict__ segs, const uint32_t* __restrict__ tile_seg,
            const uint32_t* __restrict__ vtiles, float* __restrict__ residue,
            const float* __restrict__ dW, uint8_t* __restrict__ msg, uint32_t* __restrict__ stage,
            uint32_t* __restrict__ tile_cnt, double* __restrict__ tile_gsum,
            float* __restrict__ bin_max_out) {
    constexpr int NCH = (THREADS / 64) * VPT;
    extern __shared__ uint32_t dyn[];
    __shared__ uint32_t ch_tot[NCH];
    TileRegs<VPT> a;
    load_tile<THREADS, VPT>(a, segs, tile_seg, vtiles, blockIdx.x, residue, dW);
    process_tile<THREADS, VPT, NTS>(a, dyn, segs, tile_seg, residue, msg, stage, tile_cnt,
                                    tile_gsum, bin_max_out, ch_tot);
}

// Long bins (L_T > 4093): one workgroup per bin, in chunks of THREADS x VPT
// float4.  The first pass finds g_max (and, for hard local selection, the
// first index holding it); the second forms G and H again, selects, compacts
// and writes the residue.  NCR > 0 (bins of at most NCR chunks): every chunk
// is loaded once, up front, and both passes run from registers (12 B per
// element exactly).  NCR = 0 (longer bins): the bin is streamed twice; the
// second pass reads what the first one just brought on chip (non-temporal:
// it is the last use), so HBM traffic stays near 12 B per element while bins
// fit the caches, and only one chunk lives in registers.
template <int THREADS, int VPT, int NCR, bool NTS>
__global__ void __launch_bounds__(THREADS)
k_tile_pass_long(const SegDev* __restrict__ segs, const uint32_t* __restrict__ tile_seg,
                 const uint32_t* __restrict__ vtiles, float* __restrict__ residue,
                 const float* __restrict__ dW, uint8_t* __restrict__ msg, uint32_t* __restrict__ stage,
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

    // One chunk's float4 (indexes past the bin clamped to its last float4,
    // so every lane loads).
    auto load_chunk = [&](uint32_t c0, f32x4 (&a)[VPT], f32x4 (&b)[VPT], auto nt) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t vi = min(c0 + uint32_t(v * THREADS + tid), tg.nvec - 1u);
            a[v] = load4<decltype(nt)::value>(residue + tg.v0 + uint64_t(vi) * 4u);
            b[v] = load4<decltype(nt)::value>(dW + tg.v0 + uint64_t(vi) * 4u);
        }
    };

    // ---- pass 1 over one chunk: largest |G| and its first index ----
    uint32_t m = 0u, mi = kSentinel;
    auto pass1 = [&](const f32x4 (&a)[VPT], const f32x4 (&b)[VPT], uint32_t c0) {
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
    };
    // largest |G| over the workgroup, ties to the lowest index
    float gm = 0.0f;
    uint32_t first = kSentinel;
    auto reduce = [&]() {
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
        gm = __uint_as_float(m);
        first = m != 0u ? mi : kSentinel;   // LS: nothing in an all-zero bin
    };

    // ---- pass 2 over one chunk: selection, compaction to staging, residue <- G ----
    uint32_t carry = 0;
    uint32_t* st = stage + tg.t0;
    auto pass2 = [&](const f32x4 (&a)[VPT], const f32x4 (&b)[VPT], uint32_t c0) {
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
                    st[r] = (g[v][c] < 0.0f ? 0x80000000u : 0u) | uint32_t(x0 + c);
                    ++r;
                }
            }
            const uint64_t e0 = tg.v0 + uint64_t(vi) * 4u;
            if (x0 >= 0 && x0 + 4 <= tlen) {
                f32x4 o;
                o.x = g[v][0]; o.y = g[v][1]; o.z = g[v][2]; o.w = g[v][3];
                store4<NTS>(residue + e0, o);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int x = x0 + c;
                    if (x >= 0 && x < tlen) residue[e0 + c] = g[v][c];
                }
            }
        }
        carry += total;
    };

    if constexpr (NCR > 0) {
        // The whole bin in registers (the launch guarantees nvec <= NCR * CV);
        // residue and dW are read once: non-temporal like the dense tile pass.
        f32x4 ra[NCR][VPT], rb[NCR][VPT];
#pragma unroll
        for (int k = 0; k < NCR; ++k) load_chunk(uint32_t(k) * CV, ra[k], rb[k], std::integral_constant<bool, kNtLoadResidue>{});
#pragma unroll
        for (int k = 0; k < NCR; ++k)
            if (uint32_t(k) * CV < tg.nvec) pass1(ra[k], rb[k], uint32_t(k) * CV);
        reduce();
#pragma unroll
        for (int k = 0; k < NCR; ++k)
            if (uint32_t(k) * CV < tg.nvec) pass2(ra[k], rb[k], uint32_t(k) * CV);   // workgroup-uniform
    } else {
        for (uint32_t c0 = 0; c0 < tg.nvec; c0 += CV) {
            f32x4 a[VPT], b[VPT];
            load_chunk(c0, a, b, std::integral_constant<bool, false>{});
            pass1(a, b, c0);
        }
        reduce();
        for (uint32_t c0 = 0; c0 < tg.nvec; c0 += CV) {
            f32x4 a[VPT], b[VPT];
            load_chunk(c0, a, b, std::integral_constant<bool, true>{});   // last use: non-temporal
            pass2(a, b, c0);
        }
    }
    if (tid == 0) {
        put_word(msg + sg.count_off + uint64_t(tg.first_bin) * sg.wb, sg.wb, carry);
        if (bin_max_out) bin_max_out[sg.bin_base + tg.first_bin] = gm;
        tile_gsum[tile] = double(gm);
        tile_cnt[tile] = carry;
    }
}

}  // namespace adacomp
