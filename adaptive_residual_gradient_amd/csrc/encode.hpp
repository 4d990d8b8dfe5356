// Compress, survivor offsets, scale, message header and encode for gfx950.
//
// Method: "AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
// page, definition paragraph and Mechanism claim on local-bin soft threshold
// and mean-g_max quantization (Algorithm 2); word widths from its Application
// claim (Table 2).
#pragma once

#include "common.hpp"

namespace adacomp {

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one value per thread (256 threads).
// ---------------------------------------------------------------------------
template <int THREADS>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds_w,
                                                         uint32_t* total) {
    constexpr int NW = THREADS / 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint32_t inc = wave_incl_add(v);
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

// The float64 sum of a scan chunk's tile sums (tiles [tb, tb + n), 1 <= n
// <= 1024) in the one fixed order every compress path uses: partial v
// (0..255) adds tiles 4v..4v+3 in order; the partials 64q..64q+63 are
// reduced by an xor butterfly over a wavefront (lane 0's result is used);
// the four results are added in order q = 0, 1, 2, 3.  Every term is >= +0,
// so adding +0.0 in place of a missing tile changes nothing.
__device__ __forceinline__ double chunk_partial(const double* __restrict__ tile_gsum, uint32_t tb,
                                                uint32_t n, uint32_t v) {
    double gs = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = v * 4u + i;
        const double x = tile_gsum[tb + min(t, n - 1u)];   // branch-free: clamped, then dropped
        gs += t < n ? x : 0.0;
    }
    return gs;
}
__device__ __forceinline__ double wave_xor_sum(double gs) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) gs += __shfl_xor(gs, d);
    return gs;
}
__device__ __forceinline__ double combine4(double a, double b, double c, double d) {
    return ((a + b) + c) + d;
}
// The same sum by one thread for a chunk of at most 32 tiles.  Partials
// 8..255 are then +0.0, so the butterfly levels 32, 16 and 8 add +0.0 to
// lanes 0..7 and the results of wavefronts 1..3 are +0.0: all exact.  What
// remains for lane 0 is levels 4, 2, 1 over partials 0..7, i.e. the fold
// a[i] += a[i + d] for d = 4, 2, 1 and i < d (the same binary tree; a sum
// of two doubles does not depend on the order of its operands).
__device__ __forceinline__ double chunk_sum_short(const double* __restrict__ tile_gsum,
                                                  uint32_t tb, uint32_t n) {
    double a[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) a[v] = chunk_partial(tile_gsum, tb, n, uint32_t(v));
#pragma unroll
    for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
        for (int i = 0; i < d; ++i) a[i] = a[i] + a[i + d];
    return a[0];
}
constexpr uint32_t kShortChunkTiles = 32;

// Chunk scan of scan chunk c by one block of 256 threads: tiles
// [chunk_tile_begin[c], chunk_tile_begin[c+1]) <= 1024.  lw: 4 LDS words,
// lg: 4 LDS doubles.
__device__ __forceinline__ void chunk_scan_block(uint32_t c, const uint32_t* __restrict__ chunk_tile_begin,
                                                 const uint32_t* __restrict__ tile_cnt,
                                                 const double* __restrict__ tile_gsum,
                                                 uint32_t* __restrict__ tile_off,
                                                 uint32_t* __restrict__ chunk_cnt,
                                                 double* __restrict__ chunk_gsum, uint32_t* lw,
                                                 double* lg) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint32_t tb = chunk_tile_begin[c], n = chunk_tile_begin[c + 1] - tb;
    uint32_t cnt[4];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = uint32_t(tid) * 4u + i;
        cnt[i] = t < n ? tile_cnt[tb + t] : 0u;
        mine += cnt[i];
    }
    double gs = chunk_partial(tile_gsum, tb, n, uint32_t(tid));
    uint32_t total;
    uint32_t run = block_exclusive_scan<256>(mine, lw, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = uint32_t(tid) * 4u + i;
        if (t < n) tile_off[tb + t] = run;
        run += cnt[i];
    }
    gs = wave_xor_sum(gs);
    if (lane == 0) lg[wv] = gs;
    __syncthreads();
    if (tid == 0) {
        chunk_cnt[c] = total;
        chunk_gsum[c] = combine4(lg[0], lg[1], lg[2], lg[3]);
    }
}

__global__ void __launch_bounds__(256)
k_chunk_scan(const uint32_t* __restrict__ chunk_tile_begin, const uint32_t* __restrict__ tile_cnt,
             const double* __restrict__ tile_gsum, uint32_t* __restrict__ tile_off,
             uint32_t* __restrict__ chunk_cnt, double* __restrict__ chunk_gsum) {
    __shared__ uint32_t lw[4];
    __shared__ double lg[4];
    chunk_scan_block(blockIdx.x, chunk_tile_begin, tile_cnt, tile_gsum, tile_off, chunk_cnt,
                     chunk_gsum, lw, lg);
}

// Finalize, by one block of 256 threads: s and survivor totals per segment,
// chunk bases, entry regions, and (write_msg) the directory, header and
// padding bytes of the message.  lsz, lns: 4 LDS words (64-bit) each.
__device__ __forceinline__ void finalize_block(const SegDev* __restrict__ segs, uint32_t nseg,
                                               uint32_t plan_hash, uint64_t entries_begin,
                                               const uint32_t* __restrict__ chunk_cnt,
                                               const double* __restrict__ chunk_gsum,
                                               uint32_t* __restrict__ chunk_base,
                                               float* __restrict__ seg_s,
                                               uint32_t* __restrict__ seg_nsurv,
                                               uint64_t* __restrict__ seg_eoff,
                                               uint64_t* __restrict__ seg_sbase,
                                               uint8_t* __restrict__ msg, uint64_t* lsz,
                                               uint64_t* lns, bool write_msg = true) {
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
        if (write_msg)
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
            if (write_msg) {
                uint8_t* d = msg + 32 + 16 * uint64_t(l);
                *reinterpret_cast<float*>(d) = seg_s[l];
                *reinterpret_cast<uint32_t*>(d + 4) = uint32_t(ns);
                *reinterpret_cast<uint64_t*>(d + 8) = eoff;
                const uint64_t wend = eoff + ns * segs[l].wb;
                for (uint64_t p = wend; p < eoff + sz; ++p) msg[p] = 0;
            }
        }
        carry += asz;
        surv += ans;
    }
    if (tid == 0 && write_msg) {
        *reinterpret_cast<uint32_t*>(msg) = 0x43414441u;
        *reinterpret_cast<uint16_t*>(msg + 4) = 1;
        *reinterpret_cast<uint16_t*>(msg + 6) = 0;
        *reinterpret_cast<uint32_t*>(msg + 8) = nseg;
        *reinterpret_cast<uint32_t*>(msg + 12) = plan_hash;
        *reinterpret_cast<uint64_t*>(msg + 16) = entries_begin + carry;
        *reinterpret_cast<uint64_t*>(msg + 24) = surv;
    }
    if (tid == 0) seg_sbase[nseg] = surv;
}

__global__ void __launch_bounds__(256)
k_finalize(const SegDev* __restrict__ segs, uint32_t nseg, uint32_t plan_hash,
           uint64_t entries_begin, const uint32_t* __restrict__ chunk_cnt,
           const double* __restrict__ chunk_gsum, uint32_t* __restrict__ chunk_base,
           float* __restrict__ seg_s, uint32_t* __restrict__ seg_nsurv,
           uint64_t* __restrict__ seg_eoff, uint64_t* __restrict__ seg_sbase,
           uint8_t* __restrict__ msg) {
    __shared__ uint64_t lsz[4], lns[4];
    finalize_block(segs, nseg, plan_hash, entries_begin, chunk_cnt, chunk_gsum, chunk_base, seg_s,
                   seg_nsurv, seg_eoff, seg_sbase, msg, lsz, lns);
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
// Survivor rounds per batch; the next batch's staged keys are in flight while
// this batch's G values are read, so two batches' tables live in registers.
constexpr int kEncBatch = 4;
// 2048 wavefronts, 8 per CU.  Against 8192, this shortens the launch and the
// finalize step every workgroup repeats (a 25 M-element, 0.36 M-survivor
// table: finish 23 -> 15 us); finishes bound by their scattered residue
// stores (1.07e9 elements, or 10% of elements sent) took the same time.
constexpr uint32_t kEncMaxBlocks = 512;

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

// Wavefront w of W: its share of the survivors (wavefront-uniform arguments).
__device__ __forceinline__ void encode_wave(uint32_t w, uint32_t W, const SegDev* __restrict__ segs,
                                            uint32_t nseg, const uint32_t* __restrict__ tile_seg,
                                            const uint32_t* __restrict__ stage,
                                            const uint32_t* __restrict__ tile_cnt,
                                            const uint32_t* __restrict__ tile_off,
                                            const uint32_t* __restrict__ chunk_base,
                                            const float* __restrict__ seg_s,
                                            const uint64_t* __restrict__ seg_eoff,
                                            const uint64_t* __restrict__ seg_sbase,
                                            uint8_t* __restrict__ msg, float* __restrict__ residue,
                                            uint32_t ntiles) {
    const uint32_t lane = threadIdx.x & 63u;
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
        uint32_t ltwb = 0, mag = 0, gofs = kSentinel;
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
            // k_tile_pass stages each survivor's G after the tile's keys when both fit
            const uint32_t full = cnt + skip;
            if (q.ct.variant != 2u && 2u * full <= tg.tlen) gofs = full;
        }
        // Survivors base + 64u + lane (u < kEncBatch), clamped to the last one: owning lane,
        // rank in the owner's tile, the tile's first element, the staged key and, where it
        // was staged, G (staged[u]).
        struct Batch {
            uint32_t own[kEncBatch], k[kEncBatch], key[kEncBatch];
            uint64_t tt[kEncBatch];
            float g[kEncBatch];
            bool staged[kEncBatch];
        };
        auto issue = [&](uint32_t base, Batch& b) {
#pragma unroll
            for (int u = 0; u < kEncBatch; ++u) {
                const uint32_t e = min(base + 64u * u + lane, take - 1u);
                uint32_t L = 0;   // lanes whose survivors all precede e
#pragma unroll
                for (uint32_t bit = 32; bit >= 1; bit >>= 1)
                    if (__shfl(incl, int(L + bit - 1u)) <= e) L += bit;
                b.own[u] = L;
                b.k[u] = e - __shfl(excl, int(L));
                b.tt[u] = (uint64_t(__shfl(uint32_t(t0 >> 32), int(L))) << 32) |
                          __shfl(uint32_t(t0), int(L));
                const uint32_t rk = (L == 0 ? r0 : 0u) + b.k[u], go = __shfl(gofs, int(L));
                b.key[u] = stage[b.tt[u] + rk];
                b.staged[u] = go != kSentinel;
                b.g[u] = b.staged[u] ? __uint_as_float(stage[b.tt[u] + go + rk]) : 0.0f;
            }
        };
        if (take != 0) {   // wavefront-uniform; the window advances below either way
            // One round trip per batch where G was staged with the keys, else two (the keys,
            // then G at those elements): the next batch's keys are requested (always,
            // clamped) while this batch's G is in flight.
            Batch cur;
            issue(0, cur);
            for (uint32_t base = 0; base < take; base += 64u * kEncBatch) {   // wavefront-uniform
                // G of every survivor of the batch (the tile pass left residue = G there).
                float gq[kEncBatch];
#pragma unroll
                for (int u = 0; u < kEncBatch; ++u)
                    gq[u] = cur.staged[u] ? cur.g[u] : residue[cur.tt[u] + (cur.key[u] & 0x7FFFFFFFu)];
                Batch nxt;
                issue(base + 64u * kEncBatch, nxt);
#pragma unroll
                for (int u = 0; u < kEncBatch; ++u) {
                    const uint32_t L = cur.own[u];
                    const uint64_t ea = (uint64_t(__shfl(uint32_t(eat >> 32), int(L))) << 32) |
                                        __shfl(uint32_t(eat), int(L));
                    const uint32_t lw = __shfl(ltwb, int(L)), mg = __shfl(mag, int(L));
                    const float sv = __shfl(s, int(L));
                    if (base + 64u * u + lane < take) {
                        const uint32_t lt = lw >> 2, wb = lw & 3u;
                        const uint32_t x = cur.key[u] & 0x7FFFFFFFu;
                        const uint32_t neg = cur.key[u] >> 31;
                        const uint32_t bin = div_bin(x, lt, mg);
                        const uint32_t topbit = wb == 1u ? 7u : 15u;
                        put_word(msg + ea + uint64_t(cur.k[u]) * wb, wb, (neg << topbit) | (x - bin * lt));
                        const float gv = gq[u];
                        // residue <- G - G_q with G_q = sign(G) * s
                        residue[cur.tt[u] + x] = neg ? gv + sv : gv - sv;
                    }
                }
                cur = nxt;
            }
        }
        remaining -= take;
        tile0 += 64u;
        r0 = 0;
    }
}

__global__ void __launch_bounds__(256)
k_encode(const SegDev* __restrict__ segs, uint32_t nseg, const uint32_t* __restrict__ tile_seg,
         const uint32_t* __restrict__ stage, const uint32_t* __restrict__ tile_cnt,
         const uint32_t* __restrict__ tile_off, const uint32_t* __restrict__ chunk_base,
         const float* __restrict__ seg_s, const uint64_t* __restrict__ seg_eoff,
         const uint64_t* __restrict__ seg_sbase, uint8_t* __restrict__ msg,
         float* __restrict__ residue, uint32_t ntiles) {
    encode_wave(blockIdx.x * 4u + (threadIdx.x >> 6), gridDim.x * 4u, segs, nseg, tile_seg, stage,
                tile_cnt, tile_off, chunk_base, seg_s, seg_eoff, seg_sbase, msg, residue, ntiles);
}

// ---------------------------------------------------------------------------
// Finalize + encode in one kernel (tables whose scan-chunk and segment tables
// fit in LDS): every workgroup loads the chunk survivor counts and sums of
// bin maxima, runs the finalize step on LDS arrays (workgroup 0 also writes
// the directory, header and padding) and encodes its share of the survivors
// with the segment and chunk levels of the search in LDS.  Same functions,
// same order as k_finalize + k_encode, so the same bytes.
// ---------------------------------------------------------------------------
struct ChunkFinishArgs {
    const SegDev* segs;
    const uint32_t* tile_seg;
    const uint32_t* stage;
    const uint32_t* tile_cnt;
    const uint32_t* tile_off;
    const uint32_t* chunk_cnt;
    const double* chunk_gsum;
    uint8_t* msg;
    float* residue;
    uint64_t entries_begin;
    uint32_t nchunks;
    uint32_t nseg;
    uint32_t ntiles;
    uint32_t plan_hash;
};

__global__ void __launch_bounds__(256) k_finish_chunks(ChunkFinishArgs A) {
    extern __shared__ uint64_t dyn64[];   // 8-byte aligned
    __shared__ uint64_t lsz[4], lns[4];
    const uint32_t C = A.nchunks, S = A.nseg;
    // [C] chunk sums, [S] entry offsets, [S + 1] survivors before each
    // segment (64-bit); [C] chunk counts, [C] chunk bases, [S] s, [S] survivors.
    double* cgs = reinterpret_cast<double*>(dyn64);
    uint64_t* seoff = reinterpret_cast<uint64_t*>(cgs + C);
    uint64_t* ssbase = seoff + S;
    uint32_t* ccnt = reinterpret_cast<uint32_t*>(ssbase + S + 1);
    uint32_t* cbase = ccnt + C;
    float* ss = reinterpret_cast<float*>(cbase + C);
    uint32_t* sn = reinterpret_cast<uint32_t*>(ss + S);
    for (uint32_t c = threadIdx.x; c < C; c += 256) {
        ccnt[c] = A.chunk_cnt[c];
        cgs[c] = A.chunk_gsum[c];
    }
    __syncthreads();
    finalize_block(A.segs, S, A.plan_hash, A.entries_begin, ccnt, cgs, cbase, ss, sn, seoff, ssbase,
                   A.msg, lsz, lns, blockIdx.x == 0);
    __syncthreads();
    encode_wave(blockIdx.x * 4u + (threadIdx.x >> 6), gridDim.x * 4u, A.segs, S, A.tile_seg, A.stage,
                A.tile_cnt, A.tile_off, cbase, ss, seoff, ssbase, A.msg, A.residue, A.ntiles);
}

}  // namespace adacomp
