// Decode-accumulate kernels for gfx950.
//
// Method: "AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
// page, definition paragraph and Mechanism claim on local-bin soft threshold
// and mean-g_max quantization (Algorithm 2); word widths from its Application
// claim (Table 2).
#pragma once

#include "common.hpp"

namespace adacomp {

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
    uint64_t* drec;       // [K*P]: entry records of the LDS decode tiles (k_decode_records)
};

// An entry record: the byte address of a decode tile's first entry word in a
// message (device addresses fit 48 bits) and the number of the tile's
// entries in that message (at most a tile's 4096 elements) in the top 16
// bits; 0 for a tile without entries and for a refused message.
constexpr uint64_t kRecAddrMask = (uint64_t(1) << 48) - 1u;

// What a message must satisfy before any byte past its header is read: the
// plan's magic, version, layer count and table hash, and a total length
// between the end of the count regions and the plan's capacity, a multiple
// of 16.  Every count word then lies inside the message.
struct MsgGeom {
    uint32_t nseg;
    uint32_t plan_hash;
    uint64_t entries_begin;   // end of the count regions
    uint64_t capacity;        // largest message of the plan
};

__device__ __forceinline__ bool header_matches(const uint8_t* m, const MsgGeom& g) {
    const uint64_t total = *reinterpret_cast<const uint64_t*>(m + 16);
    return *reinterpret_cast<const uint32_t*>(m) == 0x43414441u &&
           *reinterpret_cast<const uint16_t*>(m + 4) == 1 &&
           *reinterpret_cast<const uint32_t*>(m + 8) == g.nseg &&
           *reinterpret_cast<const uint32_t*>(m + 12) == g.plan_hash &&
           total >= g.entries_begin && total <= g.capacity && (total & 15u) == 0u;
}

// A chunk total with this bit set: some tile of the chunk counts more
// transmitted elements than it has elements (a corrupt message).
constexpr uint32_t kChunkBad = 0x80000000u;

// Sum of the count words in message bytes [a0, a1), read as the aligned
// 16-byte blocks that cover them (count regions start 16-byte aligned and
// are zero-padded to 16 bytes, so those blocks lie inside the message).
__device__ __forceinline__ uint32_t sum_count_words(const uint8_t* m, uint64_t a0, uint64_t a1,
                                                    uint32_t wb) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4* gu4;
    uint32_t s = 0;
    for (uint64_t d = a0 & ~uint64_t(15); d < a1; d += 16) {
        const u32x4 v = *(gu4)(m + d);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint64_t dj = d + 4u * uint32_t(j);
            uint32_t x = w4[j];
            if (dj + 4 <= a0 || dj >= a1) {
                x = 0;   // no byte of [a0, a1)
            } else {
                if (dj < a0) x &= ~0u << (8u * uint32_t(a0 - dj));          // bytes before a0
                if (dj + 4 > a1) x &= ~0u >> (8u * uint32_t(dj + 4 - a1));  // bytes from a1 on
            }
            s += wb == 1u ? (x & 0xFFu) + ((x >> 8) & 0xFFu) + ((x >> 16) & 0xFFu) + (x >> 24)
                          : (x & 0xFFFFu) + (x >> 16);
        }
    }
    return s;
}

// The same with the tile's blocks requested together when they are at most
// NB (one memory round trip instead of one per block; the addresses are
// clamped to the tile's last block, so every load stays inside the message).
template <int NB>
__device__ __forceinline__ uint32_t sum_count_words_batched(const uint8_t* m, uint64_t a0, uint64_t a1,
                                                            uint32_t wb) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4* gu4;
    const uint64_t d0 = a0 & ~uint64_t(15);
    const uint32_t nblk = uint32_t((a1 - d0 + 15u) >> 4);
    if (nblk > uint32_t(NB)) return sum_count_words(m, a0, a1, wb);
    u32x4 v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) v[i] = *(gu4)(m + d0 + 16u * min(uint32_t(i), nblk - 1u));
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint64_t dj = d0 + 16u * uint32_t(i) + 4u * uint32_t(j);
            uint32_t x = uint32_t(i) < nblk ? w4[j] : 0u;
            if (dj + 4 <= a0 || dj >= a1) {
                x = 0;   // no byte of [a0, a1)
            } else {
                if (dj < a0) x &= ~0u << (8u * uint32_t(a0 - dj));          // bytes before a0
                if (dj + 4 > a1) x &= ~0u >> (8u * uint32_t(dj + 4 - a1));  // bytes from a1 on
            }
            s += wb == 1u ? (x & 0xFFu) + ((x >> 8) & 0xFFu) + ((x >> 16) & 0xFFu) + (x >> 24)
                          : (x & 0xFFFFu) + (x >> 16);
        }
    }
    return s;
}

// Per (chunk of decode tiles, message): survivors of each decode tile from
// the count words, offsets within the chunk, chunk totals.  Thread t takes
// tiles t, t + 256, t + 512, t + 768 (decode chunks hold at most
// kDecChunkTiles = 256 tiles: one round), so the lanes of a wavefront read
// neighbouring tiles' count words together; one block scan per round of
// 256 tiles gives the offsets in tile order.  NB > 0: a tile's count blocks
// are requested together when they are at most NB (tables whose decode
// tiles hold many count words: dense short bins); NB = 0: one at a time.
template <int NB>
__global__ void __launch_bounds__(256)
k_decode_count(MsgPtrs msgs, const CountChunk* __restrict__ chunks, uint32_t DT, uint32_t DC,
               MsgGeom geo, DecodeWs ws) {
    __shared__ uint32_t lw[4];
    __shared__ uint32_t bad;
    const uint32_t c = blockIdx.x, k = blockIdx.y;
    const uint8_t* m = msgs.p[k];
    if (threadIdx.x == 0) {
        bad = 0;
        if (c == 0 && k == 0) *ws.status = 0;   // k_decode_base counts the rejected messages
    }
    // A message made for another table is never read past its header.
    const bool ok = header_matches(m, geo);
    const CountChunk cc = chunks[c];
    const uint32_t tb = cc.tile0, n = cc.ntiles;
    __syncthreads();   // bad is cleared before any thread sets it
    uint32_t cnt[4];
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = uint32_t(i) * 256u + threadIdx.x;
        uint32_t s = 0;
        if (ok && t < n) {
            const uint32_t first_bin = cc.first_bin + t * cc.bpt;
            const uint32_t nb = min(cc.bpt, cc.nbins - first_bin);
            const uint64_t a0 = cc.count_off + uint64_t(first_bin) * cc.wb;
            s = NB > 0 ? sum_count_words_batched<(NB > 0 ? NB : 1)>(m, a0, a0 + uint64_t(nb) * cc.wb, cc.wb)
                       : sum_count_words(m, a0, a0 + uint64_t(nb) * cc.wb, cc.wb);
            // A tile never sends more elements than it holds.
            const uint64_t e0 = uint64_t(first_bin) * cc.lt;
            const uint64_t elems = min(uint64_t(nb) * cc.lt, cc.numel - e0);
            if (s > elems) {
                over = true;
                s = 0;
            }
        }
        cnt[i] = s;
    }
    if (over) atomicOr(&bad, 1u);
    uint32_t base = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (uint32_t(i) * 256u >= n) break;   // workgroup-uniform: no tile left in the chunk
        const uint32_t t = uint32_t(i) * 256u + threadIdx.x;
        uint32_t total;
        const uint32_t ex = block_exclusive_scan<256>(cnt[i], lw, &total);
        if (t < n) {
            ws.dcnt[uint64_t(k) * DT + tb + t] = cnt[i];
            ws.doff[uint64_t(k) * DT + tb + t] = base + ex;
        }
        base += total;
    }
    __syncthreads();
    if (threadIdx.x == 0) ws.dchunk_cnt[uint64_t(k) * DC + c] = base | (bad ? kChunkBad : 0u);
}

// One block per message: per-segment s and entry offsets, chunk bases, and
// the message's validity.  A message is decoded only if its header matches
// (header_matches) and, for every segment, its directory entry is
// consistent with the count words: entry offset 16-byte aligned and at or
// past the count regions, survivors at most the segment's elements and equal
// to the sum of its count words, no tile counting more than it holds, and
// the entry region (padded to 16 bytes) inside the message's total length.
// Then every entry word a decode kernel reads lies inside the message.  A
// rejected message contributes nothing and is counted in the status word
// (reset by k_decode_count).
__global__ void __launch_bounds__(256)
k_decode_base(MsgPtrs msgs, uint32_t K, const SegDev* __restrict__ segs, MsgGeom geo,
              uint32_t DC, DecodeWs ws) {
    __shared__ uint32_t fail;
    const uint32_t k = blockIdx.x;
    const uint8_t* m = msgs.p[k];
    if (threadIdx.x == 0) fail = header_matches(m, geo) ? 0u : 1u;
    __syncthreads();
    const bool hdr_ok = fail == 0u;
    const uint64_t total = hdr_ok ? *reinterpret_cast<const uint64_t*>(m + 16) : 0u;
    bool bad = false;
    for (uint32_t l = threadIdx.x; l < geo.nseg; l += 256) {
        const uint64_t i = uint64_t(k) * geo.nseg + l;
        const SegDev sg = segs[l];
        float s = 0.0f;
        uint64_t eoff = 0;
        uint32_t nsurv = 0;
        if (hdr_ok) {
            const uint8_t* d = m + 32 + 16 * uint64_t(l);
            s = *reinterpret_cast<const float*>(d);
            nsurv = *reinterpret_cast<const uint32_t*>(d + 4);
            eoff = *reinterpret_cast<const uint64_t*>(d + 8);
            bad |= (eoff & 15u) != 0u || eoff < geo.entries_begin || uint64_t(nsurv) > sg.numel ||
                   eoff > total || rup16(uint64_t(nsurv) * sg.wb) > total - eoff;
        }
        ws.dseg_s[i] = s;
        ws.dseg_eoff[i] = eoff;
        const uint64_t c0 = uint64_t(k) * DC + sg.dt.chunk_begin;
        uint64_t run = 0;
        // Chunk totals sixteen at a time, all requested before any is used.
        for (uint32_t c = 0; c < sg.dt.nchunks; c += 16) {
            uint32_t v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = c + u < sg.dt.nchunks ? ws.dchunk_cnt[c0 + c + u] : 0u;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (c + u < sg.dt.nchunks) ws.dchunk_base[c0 + c + u] = uint32_t(run);
                bad |= (v[u] & kChunkBad) != 0u;
                run += v[u] & ~kChunkBad;
            }
        }
        if (hdr_ok) bad |= run != nsurv;
    }
    if (bad) atomicOr(&fail, 1u);
    __syncthreads();
    if (threadIdx.x == 0) {
        ws.dvalid[k] = fail == 0u ? 1u : 0u;
        if (fail) atomicAdd(ws.status, 1u);
    }
}

// Per (message, LDS decode tile in launch order): the tile's entry record,
// so that k_decode_tiles requests its entry words in the same round trip as
// its count words.  Thread p takes launch position p; the message loop is
// unrolled by four so that each round's loads are in flight together.
__global__ void __launch_bounds__(256)
k_decode_records(MsgPtrs msgs, uint32_t K, const DecDesc* __restrict__ descs, uint32_t P,
                 uint32_t DT, uint32_t DC, uint32_t nseg, DecodeWs ws) {
    const uint32_t p = blockIdx.x * 256u + threadIdx.x;
    if (p >= P) return;
    const DecDesc dd = descs[p];
    for (uint32_t k0 = 0; k0 < K; k0 += 4) {
        uint32_t n[4], cb[4], off[4], ok[4];
        uint64_t eoff[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t k = min(k0 + uint32_t(u), K - 1u);
            ok[u] = ws.dvalid[k];
            n[u] = ws.dcnt[uint64_t(k) * DT + dd.tile];
            off[u] = ws.doff[uint64_t(k) * DT + dd.tile];
            cb[u] = ws.dchunk_base[uint64_t(k) * DC + dd.chunk];
            eoff[u] = ws.dseg_eoff[uint64_t(k) * nseg + dd.si];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t k = k0 + uint32_t(u);
            if (k >= K) break;
            uint64_t r = 0;
            if (ok[u] != 0u && n[u] != 0u) {
                const uint64_t a = reinterpret_cast<uint64_t>(msgs.p[k]) + eoff[u] +
                                   (uint64_t(cb[u]) + off[u]) * dd.wb;
                r = (a & kRecAddrMask) | (uint64_t(n[u]) << 48);
            }
            ws.drec[uint64_t(k) * P + p] = r;
        }
    }
}

// Index word at byte address a (w = 8 or 16 bits), read as the aligned
// 16-bit word that contains it; messages are 16-byte aligned and padded to a
// multiple of 16 bytes, so the read stays inside the message.
// The address is formed from integers kept in LDS, so it is cast to a
// global-address-space pointer (a global load, not a flat one).
typedef const __attribute__((address_space(1))) uint16_t* global_u16_ptr;
typedef const __attribute__((address_space(1))) uint32_t* global_u32_ptr;

// Entry rounds whose loads are issued together (1: 1.59 ms for the K = 16
// decode of the 1.07e9-element workload, 2: 1.50 ms, 4: 1.50 ms).
constexpr int kDecBatch = 2;

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

// Optimizer steps fused into decode, on the summed gradient, every operation
// one float32 operation rounded to nearest (no contraction):
//   SGD with momentum (no dampening, no Nesterov):
//     g = scale * sum (+ weight_decay * w),  m = beta1 * m + g,  w = w - lr * m
//   Adam with bias-corrected moments (c1 = 1 - beta1^t, c2 = 1 - beta2^t):
//     m = beta1 * m + (1 - beta1) * g,  v = beta2 * v + (1 - beta2) * (g * g),
//     w = w - lr * ((m / c1) / (sqrt(v / c2) + eps))
constexpr int kOptNone = 0, kOptSgd = 1, kOptAdam = 2;

struct OptParams {
    float lr, beta1, beta2, eps, weight_decay, scale;
    float c1, c2, omb1, omb2;   // Adam: bias corrections, 1 - beta1, 1 - beta2
    float* w;
    float* m;
    float* v;
};

template <int OPT>
__device__ __forceinline__ void opt_step(float sum, float& w, float& m, float& v, const OptParams& p) {
    float g = p.scale * sum;
    if (p.weight_decay != 0.0f) g = g + p.weight_decay * w;
    if (OPT == kOptSgd) {
        m = p.beta1 * m + g;
        w = w - p.lr * m;
    } else {
        m = p.beta1 * m + p.omb1 * g;
        v = p.beta2 * v + p.omb2 * (g * g);
        const float mh = m / p.c1;
        const float vh = v / p.c2;
        w = w - p.lr * (mh / (sqrtf(vh) + p.eps));
    }
}

// One float4 of weights and state: step the four elements and store those
// inside the tile (whole float4 when the tile covers it).
template <int OPT>
__device__ __forceinline__ void opt_apply(const f32x4& a, f32x4& wq, f32x4& mq, f32x4& vq,
                                          const OptParams& op, uint64_t e0, int x0, int tlen) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float wc = wq[c], mc = mq[c], vc = vq[c];
        opt_step<OPT>(a[c], wc, mc, vc, op);
        wq[c] = wc;
        mq[c] = mc;
        vq[c] = vc;
    }
    if (x0 >= 0 && x0 + 4 <= tlen) {
        store4<true>(op.w + e0, wq);
        store4<true>(op.m + e0, mq);
        if (OPT == kOptAdam) store4<true>(op.v + e0, vq);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int x = x0 + c;
            if (x >= 0 && x < tlen) {
                op.w[e0 + c] = wq[c];
                op.m[e0 + c] = mq[c];
                if (OPT == kOptAdam) op.v[e0 + c] = vq[c];
            }
        }
    }
}

constexpr uint32_t kOptSlots = kDecCap / 4 / 256;   // float4 per thread of an LDS tile

// OPT != kOptNone: instead of writing the tile's sums to out, the tile's
// weights and optimizer state (loaded when the tile starts, kept in
// registers) take one step.
template <int THREADS, bool LDS_ACC, int OPT = kOptNone>
__global__ void __launch_bounds__(THREADS)
k_decode_apply(MsgPtrs msgs, uint32_t K, uint32_t KG, uint32_t pstride,
               const DecDesc* __restrict__ descs, uint32_t DT, uint32_t DC, uint32_t nseg,
               DecodeWs ws, float* __restrict__ out, int accumulate, uint32_t acc_words,
               OptParams op) {
    constexpr bool FUSED = OPT != kOptNone;
    static_assert(!FUSED || LDS_ACC, "optimizer steps are fused into LDS tiles");
    // 256-thread tiles request their weights and state when the tile starts
    // (held in registers); larger tiles load them float4 by float4 at the end.
    constexpr bool PRELOAD = FUSED && THREADS == 256;
    constexpr int NW = THREADS / 64;
    extern __shared__ uint64_t dyn64[];
    uint32_t* dyn = reinterpret_cast<uint32_t*>(dyn64);
    const uint32_t accw = LDS_ACC ? (acc_words + 1u) & ~1u : 0u;   // keep 8-byte alignment
    uint64_t* mptr = reinterpret_cast<uint64_t*>(dyn + accw);   // [K] message, 0 if foreign
    uint64_t* eaddr = mptr + K;
    float* ks = reinterpret_cast<float*>(eaddr + KG);
    uint32_t* wfk_all = reinterpret_cast<uint32_t*>(ks + K);   // [NW][KG + 1]
    uint32_t* pref = wfk_all + NW * (KG + 1);             // [KG][pstride]

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // Message addresses first: they do not depend on the descriptor, so the
    // count words below wait for one round trip, not two.
    for (uint32_t k = tid; k < K; k += THREADS)
        mptr[k] = ws.dvalid[k] ? reinterpret_cast<uint64_t>(msgs.p[k]) : 0u;
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
    constexpr uint32_t NS = PRELOAD ? kOptSlots : 1;
    f32x4 wv4[NS], mv4[NS], vv4[OPT == kOptAdam ? NS : 1];
    if (PRELOAD) {   // weights and state of this thread's float4 slots, requested early
#pragma unroll
        for (uint32_t j = 0; j < NS; ++j) {
            const uint32_t vi = uint32_t(tid) + THREADS * j;
            if (vi < nvec) {
                wv4[j] = load4<true>(op.w + v0 + uint64_t(vi) * 4u);
                mv4[j] = load4<true>(op.m + v0 + uint64_t(vi) * 4u);
                if (OPT == kOptAdam) vv4[OPT == kOptAdam ? j : 0] = load4<true>(op.v + v0 + uint64_t(vi) * 4u);
            }
        }
    }
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
        // Count words of the tile's bins for this group of messages (a
        // foreign message counts nothing and is never read).
        for (uint32_t i = tid; i < kn * nb; i += THREADS) {
            const uint32_t kk = i / nb, b = i - kk * nb;
            const uint64_t mb = mptr[k0 + kk];
            pref[kk * pstride + b + 1] = mb != 0u ? word_at(mb + dd.count_at + uint64_t(b) * wb, wb) : 0u;
        }
        if (tid < int(kn)) {
            const uint32_t k = k0 + tid;
            const uint64_t base = uint64_t(ws.dchunk_base[uint64_t(k) * DC + dd.chunk]) +
                                  ws.doff[uint64_t(k) * DT + dd.tile];
            eaddr[tid] = mptr[k] + ws.dseg_eoff[uint64_t(k) * nseg + dd.si] + base * wb;
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
    if (LDS_ACC && !FUSED) {
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
    if (PRELOAD) {
        __syncthreads();
#pragma unroll
        for (uint32_t j = 0; j < NS; ++j) {
            const uint32_t vi = uint32_t(tid) + THREADS * j;
            if (vi >= nvec) continue;
            const f32x4 a = *reinterpret_cast<const f32x4*>(acc + vi * 4);
            f32x4 wq = wv4[j], mq = mv4[j], vq = vv4[OPT == kOptAdam ? j : 0];
            opt_apply<OPT>(a, wq, mq, vq, op, v0 + uint64_t(vi) * 4u, int(vi * 4) - int(lead),
                           int(tlen));
        }
    } else if (FUSED) {
        __syncthreads();
        for (uint32_t vi = tid; vi < nvec; vi += THREADS) {
            const uint64_t e0 = v0 + uint64_t(vi) * 4u;
            const f32x4 a = *reinterpret_cast<const f32x4*>(acc + vi * 4);
            f32x4 wq = load4<true>(op.w + e0), mq = load4<true>(op.m + e0), vq = {0.f, 0.f, 0.f, 0.f};
            if (OPT == kOptAdam) vq = load4<true>(op.v + e0);
            opt_apply<OPT>(a, wq, mq, vq, op, e0, int(vi * 4) - int(lead), int(tlen));
        }
    }
}

// ---------------------------------------------------------------------------
// Decode of tiles of whole bins of at most kDecCap elements (L_T <= 4093),
// 256 threads, without ordered LDS additions.
//
// Messages are taken in groups of at most kMaskMsgs.  For a group, every
// entry sets, with an LDS atomic OR, two bits in the 32-bit word of its
// element: bit kk (message kk of the group sends the element) and bit
// 16 + kk (with a negative sign).  Bits of different messages never collide,
// so the order of the atomics does not matter and every entry of the tile is
// placed in parallel.  Then the thread owning an element (float4 slots tid,
// tid + 256, ...) walks its hit bits in ascending message order and adds
// +s or -s one float32 addition at a time: the same additions, in the same
// order, as summing the messages one after the other.
//
// Entry words are read as the aligned 16-byte blocks covering each message's
// run of entries for the tile (a message's entries for a tile are contiguous:
// bin-major, ascending index), so the loads are coalesced and every lane
// gets 8 (16-bit words) or 16 (8-bit words) consecutive entries.  The bin of
// a block's first entry comes from a binary search of that message's count
// prefix over the tile's bins; the following entries advance the bin
// linearly.
//
// SEP = false (K <= kMaskMsgs, sum from +0): one LDS word per element holds
// the group's bits and is then overwritten by the element's sum (an element
// no message sends keeps 0, the bits of +0.0f).  SEP = true (more messages,
// or out += sum): a second LDS array holds each element's running sum.
// OPT != kOptNone: the sums are not written; the tile's weights and
// optimizer state (requested when the tile starts) take one step.
// ---------------------------------------------------------------------------
constexpr int kBlkBatch = 2;   // 16-byte entry blocks per thread requested together


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* global_u32x4_ptr;

// The entry words of one 16-byte block of a message's run for the tile that
// lie in the block's word window [wlo, whi): v holds the block, i0 the index
// (within the message's run for this tile) of the block's first word
// (negative when the run starts inside the block), n the run's length, pk
// the message's exclusive count prefix over the tile's bins (pk[nb] = n), wb
// the word bytes (1 or 2).  The block is shifted down to the window's first
// word in one step, then one word at a time.
template <class PK>
__device__ __forceinline__ void place_window(const u32x4& v, int i0, uint32_t wlo, uint32_t whi,
                                             uint32_t n, const PK* pk, uint32_t nb, uint32_t lt,
                                             uint32_t tlen, uint32_t lead, uint32_t wb, uint32_t hit,
                                             uint32_t* mask) {
    const uint32_t wbits = 8u * wb, top = wbits - 1u;
    const uint32_t wmask = (1u << wbits) - 1u, imask = (1u << top) - 1u;
    const int first = max(i0 + int(wlo), 0);
    const int last = min(i0 + int(whi), int(n));
    if (first >= last) return;
    // bin of the first entry: largest b < nb with pk[b] <= first
    uint32_t lo = 0, hi = nb;
    while (hi - lo > 1u) {
        const uint32_t mid = (lo + hi) >> 1;
        if (uint32_t(pk[mid]) <= uint32_t(first)) lo = mid; else hi = mid;
    }
    uint32_t b = lo, pn = pk[b + 1];
    uint64_t w0 = uint64_t(v.x) | (uint64_t(v.y) << 32), w1 = uint64_t(v.z) | (uint64_t(v.w) << 32);
    const uint32_t sbits = uint32_t(first - i0) * wbits;   // 0 .. 120
    if (sbits >= 64u) {
        w0 = w1 >> (sbits - 64u);
        w1 = 0;
    } else if (sbits != 0u) {
        w0 = (w0 >> sbits) | (w1 << (64u - sbits));
        w1 >>= sbits;
    }
#pragma unroll 1
    for (int i = first; i < last; ++i) {
        const uint32_t word = uint32_t(w0) & wmask;
        w0 = (w0 >> wbits) | (w1 << (64u - wbits));
        w1 >>= wbits;
        while (uint32_t(i) >= pn && b + 1u < nb) {
            ++b;
            pn = pk[b + 1];
        }
        const uint32_t idx = word & imask;
        const uint32_t x = b * lt + idx;
        if (idx < lt && x < tlen) atomicOr(&mask[x + lead], (word >> top) ? hit | (hit << 16) : hit);
    }
}

// The same for a window of at most 4 words, unrolled, keeping each placed
// entry's LDS slot (x + lead) in xs (kNoSlot where no entry was placed) for
// the entry-owned sums.
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;
template <class PK>
__device__ __forceinline__ void place_window4(const u32x4& v, int i0, uint32_t wlo, uint32_t whi,
                                              uint32_t n, const PK* pk, uint32_t nb, uint32_t lt,
                                              uint32_t tlen, uint32_t lead, uint32_t wb, uint32_t hit,
                                              uint32_t* mask, uint32_t (&xs)[4]) {
    const uint32_t wbits = 8u * wb, top = wbits - 1u;
    const uint32_t wmask = (1u << wbits) - 1u, imask = (1u << top) - 1u;
    const int first = max(i0 + int(wlo), 0);
    const int last = min(i0 + int(whi), int(n));
#pragma unroll
    for (int e = 0; e < 4; ++e) xs[e] = kNoSlot;
    if (first >= last) return;
    uint32_t lo = 0, hi = nb;
    while (hi - lo > 1u) {
        const uint32_t mid = (lo + hi) >> 1;
        if (uint32_t(pk[mid]) <= uint32_t(first)) lo = mid; else hi = mid;
    }
    uint32_t b = lo, pn = pk[b + 1];
    uint64_t w0 = uint64_t(v.x) | (uint64_t(v.y) << 32), w1 = uint64_t(v.z) | (uint64_t(v.w) << 32);
    const uint32_t sbits = uint32_t(first - i0) * wbits;   // 0 .. 120
    if (sbits >= 64u) {
        w0 = w1 >> (sbits - 64u);
        w1 = 0;
    } else if (sbits != 0u) {
        w0 = (w0 >> sbits) | (w1 << (64u - sbits));
        w1 >>= sbits;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = first + e;
        const uint32_t word = uint32_t(w0 >> (uint32_t(e) * wbits)) & wmask;
        if (i < last) {
            while (uint32_t(i) >= pn && b + 1u < nb) {
                ++b;
                pn = pk[b + 1];
            }
            const uint32_t idx = word & imask;
            const uint32_t x = b * lt + idx;
            if (idx < lt && x < tlen) {
                atomicOr(&mask[x + lead], (word >> top) ? hit | (hit << 16) : hit);
                xs[e] = x + lead;
            }
        }
    }
}


// The same two placements with the bins read from a table of bin starts: the
// byte of a message's run position holds b + 1 where bin b's words begin, 0
// elsewhere (the run's first position always holds a start).  An entry's bin
// is the last start at or before it, so no entry waits on a search of the
// count prefixes.
//
// The start at or before table byte P (P >= at, the run's first byte), as b + 1:
// the aligned word holding P, then, rarely, the words before it.
__device__ __forceinline__ uint32_t tbl_start_at(const uint32_t* tb32, uint32_t at, uint32_t P) {
    int q = int(P >> 2);
    uint32_t x = tb32[q] & ((P & 3u) == 3u ? ~0u : (1u << (8u * ((P & 3u) + 1u))) - 1u);
    while (true) {
        if (uint32_t(4 * q) < at) x &= ~0u << (8u * (at - uint32_t(4 * q)));   // bytes of an earlier run
        if (x != 0u || uint32_t(4 * q) <= at) break;
        --q;
        x = tb32[q];
    }
    return (x >> (8u * ((31u - __builtin_clz(x | 1u)) >> 3))) & 0xFFu;
}

__device__ __forceinline__ void place_window_tbl(const u32x4& v, int i0, uint32_t wlo, uint32_t whi,
                                                 uint32_t n, const uint32_t* tb32, uint32_t tblw, uint32_t at,
                                                 uint32_t lt, uint32_t tlen, uint32_t lead, uint32_t wb,
                                                 uint32_t hit, uint32_t* mask) {
    const int first = max(i0 + int(wlo), 0);
    const int last = min(i0 + int(whi), int(n));
    if (first >= last) return;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    // The block's start bytes: table bytes at + i0 .. at + i0 + 16 / wb - 1, read as the
    // aligned words covering them, the word indices clamped to the table (a clamped word
    // only holds bytes of words that are not placed: before the run or past its end).
    const int q0 = int(at) + i0;
    const int wq = q0 >> 2;   // floor
    const uint32_t rs = 8u * uint32_t(q0 & 3);
    uint32_t run = tbl_start_at(tb32, at, at + uint32_t(first));
    if (wb == 1u) {
        uint32_t W[5];
#pragma unroll
        for (int t = 0; t < 5; ++t) W[t] = tb32[min(max(wq + t, 0), int(tblw) - 1)];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t st = uint32_t(((uint64_t(W[g + 1]) << 32) | W[g]) >> rs);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * g + e;
                const uint32_t m = (st >> (8 * e)) & 0xFFu;
                if (i0 + j > first && m != 0u) run = m;
                const uint32_t word = (w[g] >> (8 * e)) & 0xFFu;
                const uint32_t idx = word & 0x7Fu;
                const uint32_t x = (run - 1u) * lt + idx;
                if (i0 + j >= first && i0 + j < last && idx < lt && x < tlen)
                    atomicOr(&mask[x + lead], (word >> 7) ? hit | (hit << 16) : hit);
            }
        }
    } else {
        uint32_t W[3];
#pragma unroll
        for (int t = 0; t < 3; ++t) W[t] = tb32[min(max(wq + t, 0), int(tblw) - 1)];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint32_t st = uint32_t(((uint64_t(W[g + 1]) << 32) | W[g]) >> rs);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * g + e;
                const uint32_t m = (st >> (8 * e)) & 0xFFu;
                if (i0 + j > first && m != 0u) run = m;
                const uint32_t word = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                const uint32_t idx = word & 0x7FFFu;
                const uint32_t x = (run - 1u) * lt + idx;
                if (i0 + j >= first && i0 + j < last && idx < lt && x < tlen)
                    atomicOr(&mask[x + lead], (word >> 15) ? hit | (hit << 16) : hit);
            }
        }
    }
}

// A window of at most 4 words, keeping each placed entry's LDS slot in xs.
__device__ __forceinline__ void place_window4_tbl(const u32x4& v, int i0, uint32_t wlo, uint32_t whi,
                                                  uint32_t n, const uint32_t* tb32, uint32_t at,
                                                  uint32_t lt, uint32_t tlen, uint32_t lead, uint32_t wb,
                                                  uint32_t hit, uint32_t* mask, uint32_t (&xs)[4]) {
    const uint32_t wbits = 8u * wb, top = wbits - 1u;
    const uint32_t wmask = (1u << wbits) - 1u, imask = (1u << top) - 1u;
    const int first = max(i0 + int(wlo), 0);
    const int last = min(i0 + int(whi), int(n));
#pragma unroll
    for (int e = 0; e < 4; ++e) xs[e] = kNoSlot;
    if (first >= last) return;
    uint64_t w0 = uint64_t(v.x) | (uint64_t(v.y) << 32), w1 = uint64_t(v.z) | (uint64_t(v.w) << 32);
    const uint32_t sbits = uint32_t(first - i0) * wbits;   // 0 .. 120
    if (sbits >= 64u) {
        w0 = w1 >> (sbits - 64u);
    } else if (sbits != 0u) {
        w0 = (w0 >> sbits) | (w1 << (64u - sbits));
    }
    const uint8_t* tb = reinterpret_cast<const uint8_t*>(tb32) + at;
    uint32_t st[4];
#pragma unroll
    for (int e = 1; e < 4; ++e) st[e] = tb[min(first + e, last - 1)];
    uint32_t run = tbl_start_at(tb32, at, at + uint32_t(first));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e > 0 && st[e] != 0u) run = st[e];
        const uint32_t word = uint32_t(w0 >> (uint32_t(e) * wbits)) & wmask;
        const uint32_t idx = word & imask;
        const uint32_t x = (run - 1u) * lt + idx;
        if (first + e < last && idx < lt && x < tlen) {
            atomicOr(&mask[x + lead], (word >> top) ? hit | (hit << 16) : hit);
            xs[e] = x + lead;
        }
    }
}

template <bool SEP, int OPT, bool TBL>
__global__ void __launch_bounds__(256)
k_decode_tiles(MsgPtrs msgs, uint32_t K, uint32_t KG, uint32_t pstride,
               const DecDesc* __restrict__ descs, uint32_t DT, uint32_t DC, uint32_t nseg,
               DecodeWs ws, float* __restrict__ out, int accumulate, uint32_t acc_words,
               OptParams op, uint32_t tblw) {
    constexpr int THREADS = 256, NW = THREADS / 64;
    constexpr uint32_t NS = kDecCap / 4 / THREADS;   // float4 slots per thread
    constexpr bool FUSED = OPT != kOptNone;
    extern __shared__ f32x4 dyn4[];
    const uint32_t accw = (acc_words + 3u) & ~3u;
    uint32_t* mask = reinterpret_cast<uint32_t*>(dyn4);          // [accw]
    float* sums = reinterpret_cast<float*>(mask + accw);         // [accw] with SEP
    uint64_t* mptr = reinterpret_cast<uint64_t*>(mask + accw * (SEP ? 2u : 1u));   // [K]
    uint64_t* abase = mptr + K;                                  // [KG]
    uint32_t* nent = reinterpret_cast<uint32_t*>(abase + KG);    // [KG]
    float* ks = reinterpret_cast<float*>(nent + KG);             // [KG]
    // [KG][pstride], 16 bits each (a prefix counts at most a tile's 4096 elements)
    uint16_t* pref = reinterpret_cast<uint16_t*>(ks + KG);
    // In the same place, when a group's table is used: the bin starts of the group's runs,
    // run after run ([4 tblw] bytes, zero before the starts are written).
    uint32_t* tbl32 = reinterpret_cast<uint32_t*>(pref);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const DecDesc dd = descs[blockIdx.x];
    const uint64_t v0 = dd.t0 & ~uint64_t(3);
    const uint32_t lead = uint32_t(dd.t0 - v0);
    const uint32_t nvec = (lead + dd.tlen + 3u) >> 2;
    const uint32_t nb = dd.nb, tlen = dd.tlen, wb = dd.wb, lt = dd.lt;
    // Message addresses (0 for a rejected message; K <= THREADS): both words
    // requested together, without a branch, in the descriptor's round trip.
    if (tid < int(K)) {
        const uint64_t p = reinterpret_cast<uint64_t>(msgs.p[tid]);
        const uint32_t ok = ws.dvalid[tid];
        mptr[tid] = p & (uint64_t(0) - uint64_t(ok != 0u));
    }
    // An always readable address for loads whose result is not used.
    const uint64_t dummy = reinterpret_cast<uint64_t>(ws.dvalid);

    // This thread's float4 slots: starting values (out for out += sum) or
    // weights and optimizer state, requested now.
    f32x4 init[SEP ? NS : 1], wq[FUSED ? NS : 1], mq[FUSED ? NS : 1], vq[OPT == kOptAdam ? NS : 1];
#pragma unroll
    for (uint32_t j = 0; j < NS; ++j) {
        const uint32_t vi = uint32_t(tid) + THREADS * j;
        const uint64_t e0 = v0 + uint64_t(vi) * 4u;
        const int x0 = int(vi * 4) - int(lead);
        if (SEP) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            if (accumulate && vi < nvec) {
                if (x0 >= 0 && x0 + 4 <= int(tlen)) {
                    a = load4<true>(out + e0);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (x0 + c >= 0 && x0 + c < int(tlen)) a[c] = out[e0 + c];
                }
            }
            init[SEP ? j : 0] = a;
        }
        if (FUSED && vi < nvec) {
            wq[FUSED ? j : 0] = load4<true>(op.w + e0);
            mq[FUSED ? j : 0] = load4<true>(op.m + e0);
            if (OPT == kOptAdam) vq[OPT == kOptAdam ? j : 0] = load4<true>(op.v + e0);
        }
        if (vi < accw / 4u) reinterpret_cast<u32x4*>(mask)[vi] = u32x4{0u, 0u, 0u, 0u};
    }
    if (TBL)
        for (uint32_t q = uint32_t(tid); q < tblw / 4u; q += THREADS)
            reinterpret_cast<u32x4*>(tbl32)[q] = u32x4{0u, 0u, 0u, 0u};

    f32x4 a4[SEP ? 1 : NS];   // without SEP: this thread's sums
    bool owned = false;       // entry-owned sums (sparse tiles, without SEP)
    uint32_t own_x[4] = {kNoSlot, kNoSlot, kNoSlot, kNoSlot}, own_hit = 0;
    // Without SEP there is one group (K <= KG), so the loop below is straight-line code.
    const uint32_t ngroups = SEP ? (K + KG - 1u) / KG : 1u;
    for (uint32_t g = 0; g < ngroups; ++g) {
        const uint32_t k0 = g * KG;
        const uint32_t kn = min(KG, K - k0);
        __syncthreads();   // addresses staged; the previous group is done with pref, ks and mask
        // ---- where each message's entries start, and the count words of the tile's bins ----
        // Threads 0..kn-1 request their message's entry offset, entry count and s first, so that
        // these loads and the count words below are in flight together.
        uint64_t a_off = 0, a_msg = 0;
        uint32_t a_n = 0;
        float a_s = 0.0f;
        if (tid < int(kn)) {
            const uint32_t k = k0 + uint32_t(tid);
            a_msg = mptr[k];
            if (a_msg != 0u) {
                a_off = ws.dseg_eoff[uint64_t(k) * nseg + dd.si] +
                        (uint64_t(ws.dchunk_base[uint64_t(k) * DC + dd.chunk]) +
                         ws.doff[uint64_t(k) * DT + dd.tile]) * wb;
                a_n = ws.dcnt[uint64_t(k) * DT + dd.tile];
                a_s = ws.dseg_s[uint64_t(k) * nseg + dd.si];
            }
        }
        // Every wavefront: the length of each message's run for this tile (lane kk) and where
        // it starts in the bin table.  The table is used for tiles of at most 128 bins whose
        // runs fit it; then no bin prefix is stored.
        uint32_t t_at = 0;   // lane kk: first table byte of message kk
        bool use_tbl = false;
        if (TBL && tblw != 0u && nb <= 128u) {   // uniform
            uint32_t t_n = 0;
            if (uint32_t(lane) < kn && mptr[k0 + uint32_t(lane)] != 0u)
                t_n = ws.dcnt[uint64_t(k0 + uint32_t(lane)) * DT + dd.tile];
            const uint32_t t_incl = wave_incl_add(t_n);
            t_at = t_incl - t_n;
            use_tbl = __builtin_amdgcn_readlane(t_incl, 63) <= 4u * tblw;
        }
        // Count words into registers, one lane per bin, then per-message prefixes by DPP scans.
        // Every load is issued without a branch (unused lanes read `dummy`), so that all of a
        // wavefront's loads are in flight together.
        auto count_word = [&](uint32_t kk, uint32_t b) -> uint32_t {
            const bool use = kk < kn && b < nb;
            const uint64_t mb = mptr[k0 + min(kk, kn - 1u)];
            const bool live = use && mb != 0u;
            const uint32_t w = word_at(live ? mb + dd.count_at + uint64_t(b) * wb : dummy, wb);
            return live ? w : 0u;
        };
        auto put_prefix = [&](uint32_t kk, uint32_t b, uint32_t inc) {
            if (kk < kn && b < nb) {
                pref[kk * pstride + b + 1u] = uint16_t(inc);
                if (b == 0u) pref[kk * pstride] = 0u;
            }
        };
        // Table: the start of bin b of message kk (count c, inclusive prefix inc) in the zeroed
        // table, at = the message's first table byte.
        auto put_bins = [&](uint32_t b, uint32_t c, uint32_t inc, uint32_t at) {
            if (c != 0u && at + inc - c < 4u * tblw) reinterpret_cast<uint8_t*>(tbl32)[at + inc - c] = uint8_t(b + 1u);
        };
        if (nb <= 16u) {
            // one message per row of 16 lanes: wavefront wv, row q holds message 4 wv + q
            const uint32_t kk = 4u * uint32_t(wv) + (uint32_t(lane) >> 4), b = uint32_t(lane) & 15u;
            const uint32_t w = count_word(kk, b);
            const uint32_t inc = row_incl_add(w);
            if (TBL && use_tbl) put_bins(b, w, inc, __shfl(t_at, int(min(kk, kMaskMsgs - 1u))));   // uniform branch
            else put_prefix(kk, b, inc);
        } else if (nb <= 128u) {
            // wavefront wv: messages wv + 4 m (m < 4), bins lane and 64 + lane
            uint32_t cw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                cw[u] = count_word(uint32_t(wv) + NW * uint32_t(u >> 1), 64u * uint32_t(u & 1) + uint32_t(lane));
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t kk = uint32_t(wv) + NW * uint32_t(m);
                const uint32_t lo = wave_incl_add(cw[2 * m]);
                const uint32_t hi = wave_incl_add(cw[2 * m + 1]) + __builtin_amdgcn_readlane(lo, 63);
                if (TBL && use_tbl) {
                    const uint32_t at = __builtin_amdgcn_readlane(t_at, int(min(kk, kMaskMsgs - 1u)));
                    put_bins(uint32_t(lane), cw[2 * m], lo, at);
                    put_bins(64u + uint32_t(lane), cw[2 * m + 1], hi, at);
                } else {
                    put_prefix(kk, uint32_t(lane), lo);
                    put_prefix(kk, 64u + uint32_t(lane), hi);
                }
            }
        } else {
            // long runs of short bins: per message, 8 rounds of 64 bins at a time
            for (uint32_t kk = uint32_t(wv); kk < kn; kk += NW) {
                uint32_t carry = 0;
                for (uint32_t b0 = 0; b0 < nb; b0 += 512u) {
                    uint32_t cw[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) cw[u] = count_word(kk, b0 + 64u * uint32_t(u) + uint32_t(lane));
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t inc = wave_incl_add(cw[u]) + carry;
                        put_prefix(kk, b0 + 64u * uint32_t(u) + uint32_t(lane), inc);
                        carry = __builtin_amdgcn_readlane(inc, 63);
                    }
                }
            }
        }
        if (tid < int(kn)) {
            abase[tid] = a_msg != 0u ? a_msg + a_off : 0u;
            nent[tid] = a_n;
            ks[tid] = a_s;
        }
        __syncthreads();

        // ---- entries: 16-byte blocks, spread over the workgroup ----
        {
            // lanes 0..kn-1 of every wavefront: message kk's run and its first block
            uint64_t ab = 0;
            uint32_t ne = 0, nblk = 0;
            if (uint32_t(lane) < kn) {
                ab = abase[lane];
                ne = nent[lane];
                if (ne != 0u) nblk = uint32_t(((ab + uint64_t(ne) * wb + 15u) >> 4) - (ab >> 4));
            }
            const uint32_t incl = wave_incl_add(nblk);
            const uint32_t bs = incl - nblk;               // first block of message `lane`
            const uint32_t NBT = __builtin_amdgcn_readlane(incl, 63);
            // Each block is split into 2^sh windows of 16 >> sh bytes (at least one word),
            // as many as keep the windows within one per thread: the entries of a sparse
            // tile then spread over the whole workgroup, one or two per thread, while a
            // dense tile keeps whole blocks per thread.
            uint32_t sh = 0;
            while (sh < 3u && (NBT << (sh + 1u)) <= THREADS && (16u >> (sh + 1u)) >= wb) ++sh;
            const uint32_t NU = NBT << sh, wbytes = 16u >> sh;
            // Sparse tiles (one window of at most 4 words per thread) keep the slots of their
            // entries for entry-owned sums; others sum per element afterwards.
            owned = !SEP && NU <= THREADS && wbytes <= 4u * wb;
            if (owned) {
                const uint32_t u = min(uint32_t(tid), NU - 1u);
                const uint32_t q = u >> sh;
                uint32_t kk = 0;
#pragma unroll
                for (uint32_t step = kMaskMsgs / 2u; step >= 1u; step >>= 1) {
                    const uint32_t c = kk + step;
                    const uint32_t bc = __shfl(bs, int(min(c, kMaskMsgs - 1u)));
                    if (c < kn && bc <= q) kk = c;
                }
                const uint64_t a = (uint64_t(__shfl(uint32_t(ab >> 32), int(kk))) << 32) |
                                   __shfl(uint32_t(ab), int(kk));
                const uint32_t nbk = __shfl(nblk, int(kk));
                const uint32_t rel = min(q - __shfl(bs, int(kk)), nbk - 1u);
                const uint64_t blk = nbk != 0u ? (a & ~uint64_t(15)) + 16u * uint64_t(rel)
                                               : dummy & ~uint64_t(15);
                const u32x4 v = *(global_u32x4_ptr)blk;
                const uint32_t nq = __shfl(ne, int(kk));
                const int iq = int(int64_t(blk) - int64_t(a));
                const uint32_t sq = (u & ((1u << sh) - 1u)) * wbytes;
                const uint32_t at = TBL && use_tbl ? __shfl(t_at, int(kk)) : 0u;
                own_hit = 1u << kk;
                if (uint32_t(tid) < NU) {
                    const uint32_t wsh = wb == 1u ? 0u : 1u;
                    if (TBL && use_tbl)
                        place_window4_tbl(v, iq >> wsh, sq >> wsh, (sq + wbytes) >> wsh, nq, tbl32, at, lt,
                                          tlen, lead, wb, own_hit, mask, own_x);
                    else
                        place_window4(v, iq >> wsh, sq >> wsh, (sq + wbytes) >> wsh, nq, pref + kk * pstride, nb,
                                      lt, tlen, lead, wb, own_hit, mask, own_x);
                }
            }
            // The blocks left (all of them unless owned), kBlkBatch per thread requested
            // together; TB: bins from the bin-start table (a separate copy of the loop, so
            // that the prefix-search path keeps its own registers).
            auto blocks = [&](auto tb_tag) {
                constexpr bool TB = decltype(tb_tag)::value;
                for (uint32_t u0 = owned ? NU : 0u; u0 < NU; u0 += THREADS * kBlkBatch) {   // workgroup-uniform
                    u32x4 v[kBlkBatch];
                    uint32_t kq[kBlkBatch], nq[kBlkBatch], sq[kBlkBatch], aq[kBlkBatch];
                    int iq[kBlkBatch];
#pragma unroll
                    for (int r = 0; r < kBlkBatch; ++r) {
                        if (u0 + THREADS * uint32_t(r) >= NU) break;   // workgroup-uniform
                        const uint32_t u = min(u0 + THREADS * uint32_t(r) + uint32_t(tid), NU - 1u);
                        const uint32_t q = u >> sh;
                        // The last message whose first block is at or before q (empty messages
                        // share their successor's start, so the one found holds block q): fixed
                        // steps 8, 4, 2, 1 with every lane active.  A lane shuffle reads 0 from
                        // an inactive lane, so it must not sit in a loop whose trip count differs
                        // between lanes.
                        uint32_t kk = 0;
#pragma unroll
                        for (uint32_t step = kMaskMsgs / 2u; step >= 1u; step >>= 1) {
                            const uint32_t c = kk + step;
                            const uint32_t bc = __shfl(bs, int(min(c, kMaskMsgs - 1u)));
                            if (c < kn && bc <= q) kk = c;
                        }
                        const uint64_t a = (uint64_t(__shfl(uint32_t(ab >> 32), int(kk))) << 32) |
                                           __shfl(uint32_t(ab), int(kk));
                        // kept inside message kk's blocks whatever q (a message without blocks is
                        // never found; if it were, the always readable dummy word is read instead)
                        const uint32_t nbk = __shfl(nblk, int(kk));
                        const uint32_t rel = min(q - __shfl(bs, int(kk)), nbk - 1u);
                        const uint64_t blk = nbk != 0u ? (a & ~uint64_t(15)) + 16u * uint64_t(rel)
                                                       : dummy & ~uint64_t(15);
                        v[r] = *(global_u32x4_ptr)blk;
                        kq[r] = kk;
                        nq[r] = __shfl(ne, int(kk));
                        if (TB) aq[r] = __shfl(t_at, int(kk));
                        iq[r] = int(int64_t(blk) - int64_t(a));
                        sq[r] = (u & ((1u << sh) - 1u)) * wbytes;   // the window's first byte
                    }
#pragma unroll
                    for (int r = 0; r < kBlkBatch; ++r) {
                        if (u0 + THREADS * uint32_t(r) >= NU) break;   // workgroup-uniform
                        if (u0 + THREADS * uint32_t(r) + uint32_t(tid) >= NU) continue;
                        const uint32_t kk = kq[r];
                        const uint32_t wsh = wb == 1u ? 0u : 1u;
                        if (TB)
                            place_window_tbl(v[r], iq[r] >> wsh, sq[r] >> wsh, (sq[r] + wbytes) >> wsh, nq[r],
                                             tbl32, tblw, aq[r], lt, tlen, lead, wb, 1u << kk, mask);
                        else
                            place_window(v[r], iq[r] >> wsh, sq[r] >> wsh, (sq[r] + wbytes) >> wsh, nq[r],
                                         pref + kk * pstride, nb, lt, tlen, lead, wb, 1u << kk, mask);
                    }
                }
            };
            if (TBL && use_tbl) blocks(std::integral_constant<bool, TBL>{});
            else blocks(std::false_type{});
        }
        __syncthreads();   // every bit of the group is set
        if (TBL && SEP && tblw != 0u)   // the next group's table starts from zero (nothing reads it past the barrier)
            for (uint32_t q = uint32_t(tid); q < tblw / 4u; q += THREADS)
                reinterpret_cast<u32x4*>(tbl32)[q] = u32x4{0u, 0u, 0u, 0u};

        // ---- sums: each thread its own elements, hits in message order ----
        if (!SEP && owned) {
            // Entry-owned: the entry of an element's lowest-numbered message adds all of the
            // element's hits in message order and writes the float over the bits, once every
            // entry has read its element's bits.  An element no message sends keeps 0, +0.0f.
            float r[4];
            uint32_t mine = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r[e] = 0.0f;
                if (own_x[e] != kNoSlot) {
                    const uint32_t m = mask[own_x[e]];
                    if (((m & 0xFFFFu) & (own_hit - 1u)) == 0u) {
                        mine |= 1u << e;
                        uint32_t h = m & 0xFFFFu;
                        float acc = 0.0f;
                        while (h != 0u) {
                            const uint32_t kk = __builtin_ctz(h);
                            h &= h - 1u;
                            const float s = ks[kk];
                            acc = acc + (((m >> (16u + kk)) & 1u) ? -s : s);
                        }
                        r[e] = acc;
                    }
                }
            }
            __syncthreads();   // every entry has read its element's bits
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((mine >> e) & 1u) mask[own_x[e]] = __float_as_uint(r[e]);
            __syncthreads();
#pragma unroll
            for (uint32_t j = 0; j < NS; ++j) {
                const uint32_t vi = uint32_t(tid) + THREADS * j;
                a4[j] = vi < nvec ? reinterpret_cast<const f32x4*>(mask)[vi] : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        } else if (!SEP) {
            // One group: the sums stay in registers.  An element's first hit is looked up
            // for the four elements of a slot together (four independent LDS reads); only
            // elements with more hits loop over the rest.
#pragma unroll
            for (uint32_t j = 0; j < NS; ++j) {
                const uint32_t vi = uint32_t(tid) + THREADS * j;
                u32x4 m4 = {0u, 0u, 0u, 0u};
                if (vi < nvec) m4 = reinterpret_cast<const u32x4*>(mask)[vi];
                float s1[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) s1[c] = ks[__builtin_ctz((m4[c] & 0xFFFFu) | 0x10000u) & 15u];
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t m = m4[c];
                    uint32_t h = m & 0xFFFFu;
                    const uint32_t k1 = __builtin_ctz(h | 0x10000u);
                    float acc = h != 0u ? (((m >> (16u + k1)) & 1u) ? -s1[c] : s1[c]) : 0.0f;
                    h &= h - 1u;
                    while (h != 0u) {
                        const uint32_t kk = __builtin_ctz(h);
                        h &= h - 1u;
                        const float s = ks[kk];
                        acc = acc + (((m >> (16u + kk)) & 1u) ? -s : s);
                    }
                    a[c] = acc;
                }
                a4[j] = a;
            }
        } else {
#pragma unroll
            for (uint32_t j = 0; j < NS; ++j) {
                const uint32_t vi = uint32_t(tid) + THREADS * j;
                if (vi >= nvec) continue;
                const u32x4 m4 = reinterpret_cast<const u32x4*>(mask)[vi];
                if (g == 0) reinterpret_cast<f32x4*>(sums)[vi] = init[SEP ? j : 0];
                uint32_t nz = (m4.x != 0u ? 1u : 0u) | (m4.y != 0u ? 2u : 0u) |
                              (m4.z != 0u ? 4u : 0u) | (m4.w != 0u ? 8u : 0u);
                while (nz != 0u) {
                    const uint32_t c = __builtin_ctz(nz);
                    nz &= nz - 1u;
                    const uint32_t m = c == 0u ? m4.x : c == 1u ? m4.y : c == 2u ? m4.z : m4.w;
                    const uint32_t at = vi * 4u + c;
                    float acc = sums[at];
                    uint32_t h = m & 0xFFFFu;
                    while (h != 0u) {
                        const uint32_t kk = __builtin_ctz(h);
                        h &= h - 1u;
                        const float s = ks[kk];
                        acc = acc + (((m >> (16u + kk)) & 1u) ? -s : s);
                    }
                    sums[at] = acc;
                    mask[at] = 0u;
                }
            }
        }
    }

    // ---- the tile's sums: written once, or one optimizer step ----
#pragma unroll
    for (uint32_t j = 0; j < NS; ++j) {
        const uint32_t vi = uint32_t(tid) + THREADS * j;
        if (vi >= nvec) continue;
        const uint64_t e0 = v0 + uint64_t(vi) * 4u;
        const int x0 = int(vi * 4) - int(lead);
        const f32x4 a = SEP ? reinterpret_cast<const f32x4*>(sums)[vi] : a4[SEP ? 0 : j];
        if (FUSED) {
            f32x4 w4 = wq[FUSED ? j : 0], m4 = mq[FUSED ? j : 0], q4 = vq[OPT == kOptAdam ? j : 0];
            opt_apply<OPT>(a, w4, m4, q4, op, e0, x0, int(tlen));
        } else if (x0 >= 0 && x0 + 4 <= int(tlen)) {
            store4<true>(out + e0, a);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (x0 + c >= 0 && x0 + c < int(tlen)) out[e0 + c] = a[c];
        }
    }
}

// The plain sum of at most kMaskMsgs messages from +0 (the decode of one
// data-parallel step), one LDS tile per workgroup: the same bits-then-ordered-
// sums scheme as k_decode_tiles with one group of messages, its message
// records (k_decode_records) staged at the start, and the tile's first entry
// blocks copied straight into LDS (global_load_lds) together with the count
// words, so that the tile needs two round trips to memory before its sums.
__global__ void __launch_bounds__(256)
k_decode_tiles_sum(MsgPtrs msgs, uint32_t K, uint32_t pstride, const DecDesc* __restrict__ descs,
                   uint32_t nseg, DecodeWs ws, float* __restrict__ out, uint32_t acc_words) {
    constexpr int THREADS = 256, NW = THREADS / 64;
    constexpr uint32_t NS = kDecCap / 4 / THREADS;   // float4 slots per thread
    extern __shared__ f32x4 dyn4[];
    const uint32_t accw = (acc_words + 3u) & ~3u;
    uint32_t* mask = reinterpret_cast<uint32_t*>(dyn4);                   // [accw]
    u32x4* blkbuf = reinterpret_cast<u32x4*>(mask + accw);                // [kPreBlocks]
    uint32_t* blkmeta = reinterpret_cast<uint32_t*>(blkbuf + kPreBlocks); // [kPreBlocks]
    uint64_t* gl_mp = reinterpret_cast<uint64_t*>(blkmeta + kPreBlocks);  // [K]
    uint64_t* gl_rc = gl_mp + K;                                          // [K]
    float* ks = reinterpret_cast<float*>(gl_rc + K);                      // [K]
    uint32_t* pref = reinterpret_cast<uint32_t*>(ks + K);                 // [K][pstride]
    const uint32_t k0 = 0, kn = K;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // First round trip: the tile's descriptor (read first, with scalar loads) and, staged
    // in LDS by wavefront 0 (lane l: message l; lanes past K repeat message K - 1), the
    // messages' addresses and this tile's entry records.
    const uint32_t pos = xcd_grouped(blockIdx.x, gridDim.x);   // this tile's launch position
    const DecDesc dd = descs[pos];
    if (wv == 0) {
        const uint32_t l = min(uint32_t(lane), K - 1u);
        const uint64_t mp = reinterpret_cast<uint64_t>(msgs.p[l]);
        const uint64_t rc = ws.drec[uint64_t(l) * gridDim.x + pos];
        gl_mp[l] = mp;
        gl_rc[l] = rc;
    }
    // lane l's 64-bit value, in every lane (l the same in every lane)
    auto lane64 = [](uint64_t x, uint32_t l) -> uint64_t {
        return (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x >> 32)), int(l)))) << 32) |
               uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x)), int(l)));
    };
    // lane l's 64-bit value (l per lane; every lane active)
    auto shfl64 = [](uint64_t x, uint32_t l) -> uint64_t {
        return (uint64_t(__shfl(uint32_t(x >> 32), int(l))) << 32) | __shfl(uint32_t(x), int(l));
    };
    const uint64_t v0 = dd.t0 & ~uint64_t(3);
    const uint32_t lead = uint32_t(dd.t0 - v0);
    const uint32_t nvec = (lead + dd.tlen + 3u) >> 2;
    const uint32_t nb = dd.nb, tlen = dd.tlen, wb = dd.wb, lt = dd.lt;
    // An always readable address for loads whose result is not used.
    const uint64_t dummy = reinterpret_cast<uint64_t>(ws.dvalid);
#pragma unroll
    for (uint32_t j = 0; j < NS; ++j) {
        const uint32_t vi = uint32_t(tid) + THREADS * j;
        if (vi < accw / 4u) reinterpret_cast<u32x4*>(mask)[vi] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();   // records staged
    // lanes 0..K-1 of every wavefront: message lane's address and entry record
    const uint64_t gmp = gl_mp[min(uint32_t(lane), kn - 1u)], grc = gl_rc[min(uint32_t(lane), kn - 1u)];

    // ---- second round trip: the entry words and the count words of the tile's messages ----
    // Lanes 0..kn-1 of every wavefront: message lane's run of entries for this tile.
    struct Runs {
        uint64_t ab;        // address of the run's first word
        uint32_t ne, nblk;  // its words, and the 16-byte blocks they touch
        uint32_t bs, NBT;   // the run's first block in the tile, and the tile's blocks
    };
    auto runs = [&]() -> Runs {
        Runs q{0u, 0u, 0u, 0u, 0u};
        if (uint32_t(lane) < kn) {
            q.ne = uint32_t(grc >> 48);
            q.ab = grc & kRecAddrMask;
            if (q.ne != 0u) q.nblk = uint32_t(((q.ab + uint64_t(q.ne) * wb + 15u) >> 4) - (q.ab >> 4));
        }
        const uint32_t incl = wave_incl_add(q.nblk);
        q.bs = incl - q.nblk;
        q.NBT = __builtin_amdgcn_readlane(incl, 63);
        return q;
    };

    const Runs R0 = runs();
    const uint32_t NBT = R0.NBT;
    // Each block is split into 2^sh windows of 16 >> sh bytes (at least one word),
    // as many as keep the windows within one per thread: the entries of a sparse
    // tile then spread over the whole workgroup, one or two per thread, while a
    // dense tile keeps whole blocks per thread.
    uint32_t sh = 0;
    while (sh < 3u && (NBT << (sh + 1u)) <= THREADS && (16u >> (sh + 1u)) >= wb) ++sh;
    const uint32_t NU = NBT << sh, wbytes = 16u >> sh;
    // Sparse tiles (one window of at most 4 words per thread) keep the slots of their
    // entries for entry-owned sums; others sum per element afterwards.
    const bool owned = NU <= THREADS && wbytes <= 4u * wb;

    // Block q of the tile (q < NBT): its message kk -- the last message whose first block
    // is at or before q (empty messages share their successor's start, so the one found
    // holds block q) -- by fixed steps 8, 4, 2, 1 with every lane active (a lane shuffle
    // reads 0 from an inactive lane, so it must not sit in a loop whose trip count differs
    // between lanes); its address, kept inside that message's blocks whatever q (a message
    // without blocks is never found; if it were, the always readable dummy word is read
    // instead); and meta = kk | run length << 4 | (byte index in the run of the block's
    // first byte + 16) << 17.
    struct BlkAt {
        uint64_t addr;
        uint32_t meta;
    };
    auto block_at = [&](const Runs& R, uint32_t q) -> BlkAt {
        uint32_t kk = 0;
#pragma unroll
        for (uint32_t step = kMaskMsgs / 2u; step >= 1u; step >>= 1) {
            const uint32_t c = kk + step;
            const uint32_t bc = __shfl(R.bs, int(min(c, kMaskMsgs - 1u)));
            if (c < kn && bc <= q) kk = c;
        }
        const uint64_t a = (uint64_t(__shfl(uint32_t(R.ab >> 32), int(kk))) << 32) |
                           __shfl(uint32_t(R.ab), int(kk));
        const uint32_t nbk = __shfl(R.nblk, int(kk));
        const uint32_t rel = min(q - __shfl(R.bs, int(kk)), nbk - 1u);
        BlkAt b;
        b.addr = nbk != 0u ? (a & ~uint64_t(15)) + 16u * uint64_t(rel) : dummy & ~uint64_t(15);
        b.meta = kk | (__shfl(R.ne, int(kk)) << 4) | (uint32_t(int(int64_t(b.addr) - int64_t(a)) + 16) << 17);
        return b;
    };
    // Count words into registers, one lane per bin, then per-message prefixes by DPP
    // scans.  Every load is issued without a branch (unused lanes, and messages without
    // entries in this tile, read `dummy`), so that all of a wavefront's loads are in
    // flight together; a load (the aligned 32 bits holding the word: count regions are
    // 16-byte aligned and padded, so they lie inside the message) and the word's value
    // are separate steps, so that no use of a loaded value sits between the loads.
    auto put_prefix = [&](uint32_t kk, uint32_t b, uint32_t inc) {
        if (kk < kn && b < nb) {
            pref[kk * pstride + b + 1u] = inc;
            if (b == 0u) pref[kk * pstride] = 0u;
        }
    };
    // Address of the tile's first count word in message kk, or 0 when the message
    // has no entries in this tile (kk the same in every lane of the wavefront).
    auto first_count = [&](uint32_t kk) -> uint64_t {
        const uint32_t kc = min(kk, kn - 1u);
        const uint64_t rc = lane64(grc, kc), mk = lane64(gmp, kc);
        return kk < kn && (rc >> 48) != 0u ? mk + dd.count_at : 0u;
    };
    auto count_load = [&](uint64_t first, uint32_t b) -> uint32_t {
        const uint64_t a = first != 0u && b < nb ? first + uint64_t(b) * wb : dummy;
        return *(global_u32_ptr)(a & ~uint64_t(3));
    };
    auto count_value = [&](uint64_t first, uint32_t b, uint32_t raw) -> uint32_t {
        // messages are 16-byte aligned: the word's place in the 32 bits is that of count_at + b wb
        const uint32_t sh8 = 8u * uint32_t((dd.count_at + uint64_t(b) * wb) & 3u);
        const uint32_t w = (raw >> sh8) & (wb == 1u ? 0xFFu : 0xFFFFu);
        return first != 0u && b < nb ? w : 0u;
    };
    // Bins of up to 16: one message per row of 16 lanes (wavefront wv, row q holds
    // message 4 wv + q).  Up to 128: wavefront wv holds messages wv + 4 m (m < 4), bins
    // lane and 64 + lane.  The count words of those are requested before the entry blocks
    // below; longer runs of short bins come after, 256 bins of a message at a time.
    const uint32_t kk16 = 4u * uint32_t(wv) + (uint32_t(lane) >> 4), b16 = uint32_t(lane) & 15u;
    uint64_t f16 = 0;
    uint64_t f128[4] = {0, 0, 0, 0};
    uint32_t cw[8];
    if (nb <= 16u) {
        const uint32_t kc = min(kk16, kn - 1u);
        const uint64_t rc = shfl64(grc, kc), mk = shfl64(gmp, kc);
        f16 = kk16 < kn && (rc >> 48) != 0u ? mk + dd.count_at : 0u;
        cw[0] = count_load(f16, b16);
    } else if (nb <= 128u) {
#pragma unroll
        for (int m = 0; m < 4; ++m) f128[m] = first_count(uint32_t(wv) + NW * uint32_t(m));
#pragma unroll
        for (int u = 0; u < 8; ++u) cw[u] = count_load(f128[u >> 1], 64u * uint32_t(u & 1) + uint32_t(lane));
    }
    // The tile's first kPreBlocks blocks are copied straight into LDS (no registers held
    // while they are in flight), one per lane of wavefronts 0 and 1, requested while the count
    // words are in flight, so that both arrive in one round trip.
    if (NBT != 0u && uint32_t(wv) < kPreBlocks / 64u) {   // wavefront-uniform
        const BlkAt b = block_at(R0, min(uint32_t(tid), NBT - 1u));
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)b.addr,
                                         (__attribute__((address_space(3))) void*)(blkbuf + 64u * uint32_t(wv)),
                                         16, 0, 0);
        if (uint32_t(tid) < NBT) blkmeta[tid] = b.meta;
    }
    float a_s = 0.0f;
    if (tid < int(kn)) a_s = ws.dseg_s[uint64_t(k0 + uint32_t(tid)) * nseg + dd.si];

    if (nb <= 16u) {
        put_prefix(kk16, b16, row_incl_add(count_value(f16, b16, cw[0])));
    } else if (nb <= 128u) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t kk = uint32_t(wv) + NW * uint32_t(m);
            const uint32_t lo = wave_incl_add(count_value(f128[m], uint32_t(lane), cw[2 * m]));
            const uint32_t hi = wave_incl_add(count_value(f128[m], 64u + uint32_t(lane), cw[2 * m + 1])) +
                                __builtin_amdgcn_readlane(lo, 63);
            put_prefix(kk, uint32_t(lane), lo);
            put_prefix(kk, 64u + uint32_t(lane), hi);
        }
    } else {
        for (uint32_t kk = uint32_t(wv); kk < kn; kk += NW) {
            const uint64_t f = first_count(kk);
            uint32_t carry = 0;
            for (uint32_t b0 = 0; b0 < nb; b0 += 256u) {
#pragma unroll
                for (int u = 0; u < 4; ++u) cw[u] = count_load(f, b0 + 64u * uint32_t(u) + uint32_t(lane));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t b = b0 + 64u * uint32_t(u) + uint32_t(lane);
                    const uint32_t inc = wave_incl_add(count_value(f, b, cw[u])) + carry;
                    put_prefix(kk, b, inc);
                    carry = __builtin_amdgcn_readlane(inc, 63);
                }
            }
        }
    }
    if (tid < int(kn)) ks[tid] = a_s;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the blocks copied into LDS
    __syncthreads();   // the tile's blocks, bin prefixes and s are in LDS

    // ---- the entries' bits: unit u is window u & (2^sh - 1) of block u >> sh ----
    uint32_t own_x[4] = {kNoSlot, kNoSlot, kNoSlot, kNoSlot}, own_hit = 0;
    const uint32_t wsh = wb == 1u ? 0u : 1u;
    if (owned) {   // one window per thread; owned implies NBT <= kPreBlocks, all copied
        const uint32_t q = min(uint32_t(tid), NU - 1u) >> sh;
        if (uint32_t(tid) < NU) {
            const uint32_t m = blkmeta[q];
            const uint32_t kk = m & 15u, sq = (uint32_t(tid) & ((1u << sh) - 1u)) * wbytes;
            own_hit = 1u << kk;
            place_window4(blkbuf[q], (int(m >> 17) - 16) >> wsh, sq >> wsh, (sq + wbytes) >> wsh,
                          (m >> 4) & 0x1FFFu, pref + kk * pstride, nb, lt, tlen, lead, wb, own_hit,
                          mask, own_x);
        }
    } else {
        const Runs R = runs();
        for (uint32_t u0 = 0; u0 < NU; u0 += THREADS * kBlkBatch) {   // workgroup-uniform
            u32x4 v[kBlkBatch] = {};
            uint32_t mt[kBlkBatch] = {};
#pragma unroll
            for (int r = 0; r < kBlkBatch; ++r) {
                if (u0 + THREADS * uint32_t(r) >= NU) break;   // workgroup-uniform
                const uint32_t q = min(u0 + THREADS * uint32_t(r) + uint32_t(tid), NU - 1u) >> sh;
                const BlkAt b = block_at(R, q);
                if (q < kPreBlocks) {
                    v[r] = blkbuf[q];
                    mt[r] = blkmeta[q];
                } else {
                    v[r] = *(global_u32x4_ptr)b.addr;
                    mt[r] = b.meta;
                }
            }
#pragma unroll
            for (int r = 0; r < kBlkBatch; ++r) {
                if (u0 + THREADS * uint32_t(r) >= NU) break;   // workgroup-uniform
                const uint32_t u = u0 + THREADS * uint32_t(r) + uint32_t(tid);
                if (u >= NU) continue;
                const uint32_t m = mt[r], kk = m & 15u, sq = (u & ((1u << sh) - 1u)) * wbytes;
                place_window(v[r], (int(m >> 17) - 16) >> wsh, sq >> wsh, (sq + wbytes) >> wsh,
                             (m >> 4) & 0x1FFFu, pref + kk * pstride, nb, lt, tlen, lead, wb, 1u << kk, mask);
            }
            // every lane's blocks are taken in here, also where a lane placed nothing, so that
            // no load is still counted as in flight after the loop (later writes to those
            // registers would wait for it)
#pragma unroll
            for (int r = 0; r < kBlkBatch; ++r) asm volatile("" ::"v"(v[r]));
        }
    }
    __syncthreads();   // every bit is set

    f32x4 a4[NS];   // this thread's sums
    // ---- sums: each thread its own elements, hits in message order ----
    if (owned) {
        // Entry-owned: the entry of an element's lowest-numbered message adds all of the
        // element's hits in message order and writes the float over the bits, once every
        // entry has read its element's bits.  An element no message sends keeps 0, +0.0f.
        float r[4];
        uint32_t mine = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = 0.0f;
            if (own_x[e] != kNoSlot) {
                const uint32_t m = mask[own_x[e]];
                if (((m & 0xFFFFu) & (own_hit - 1u)) == 0u) {
                    mine |= 1u << e;
                    uint32_t h = m & 0xFFFFu;
                    float acc = 0.0f;
                    while (h != 0u) {
                        const uint32_t kk = __builtin_ctz(h);
                        h &= h - 1u;
                        const float s = ks[kk];
                        acc = acc + (((m >> (16u + kk)) & 1u) ? -s : s);
                    }
                    r[e] = acc;
                }
            }
        }
        __syncthreads();   // every entry has read its element's bits
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if ((mine >> e) & 1u) mask[own_x[e]] = __float_as_uint(r[e]);
        __syncthreads();
#pragma unroll
        for (uint32_t j = 0; j < NS; ++j) {
            const uint32_t vi = uint32_t(tid) + THREADS * j;
            a4[j] = vi < nvec ? reinterpret_cast<const f32x4*>(mask)[vi] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    } else {
        // The sums stay in registers.  An element's first hit is looked up
        // for the four elements of a slot together (four independent LDS reads); only
        // elements with more hits loop over the rest.
#pragma unroll
        for (uint32_t j = 0; j < NS; ++j) {
            const uint32_t vi = uint32_t(tid) + THREADS * j;
            u32x4 m4 = {0u, 0u, 0u, 0u};
            if (vi < nvec) m4 = reinterpret_cast<const u32x4*>(mask)[vi];
            float s1[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) s1[c] = ks[__builtin_ctz((m4[c] & 0xFFFFu) | 0x10000u) & 15u];
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t m = m4[c];
                uint32_t h = m & 0xFFFFu;
                const uint32_t k1 = __builtin_ctz(h | 0x10000u);
                float acc = h != 0u ? (((m >> (16u + k1)) & 1u) ? -s1[c] : s1[c]) : 0.0f;
                h &= h - 1u;
                while (h != 0u) {
                    const uint32_t kk = __builtin_ctz(h);
                    h &= h - 1u;
                    const float s = ks[kk];
                    acc = acc + (((m >> (16u + kk)) & 1u) ? -s : s);
                }
                a[c] = acc;
            }
            a4[j] = a;
        }
    }

    // ---- the tile's sums, written once ----
    // Whole float4 first, then the tile's ragged ends; the sums stay live until the last
    // store, so that no register a store reads is reused for arithmetic (which would wait
    // for that store to complete).
#pragma unroll
    for (uint32_t j = 0; j < NS; ++j) {
        const uint32_t vi = uint32_t(tid) + THREADS * j;
        const int x0 = int(vi * 4) - int(lead);
        if (vi < nvec && x0 >= 0 && x0 + 4 <= int(tlen)) store4<true>(out + v0 + uint64_t(vi) * 4u, a4[j]);
    }
#pragma unroll
    for (uint32_t j = 0; j < NS; ++j) {
        const uint32_t vi = uint32_t(tid) + THREADS * j;
        const int x0 = int(vi * 4) - int(lead);
        if (vi < nvec && !(x0 >= 0 && x0 + 4 <= int(tlen))) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (x0 + c >= 0 && x0 + c < int(tlen)) out[v0 + uint64_t(vi) * 4u + c] = a4[j][c];
        }
    }
    asm volatile("" ::"v"(a4[0]), "v"(a4[1]), "v"(a4[2]), "v"(a4[3]));
}

// The optimizer step for long-bin decode tiles, whose sums were accumulated
// in a dense scratch buffer (same flat indexing as the weights).
template <int OPT>
__global__ void __launch_bounds__(256)
k_opt_tiles(const DecDesc* __restrict__ descs, const float* __restrict__ sums, OptParams op) {
    const DecDesc dd = descs[blockIdx.x];
    const uint64_t v0 = dd.t0 & ~uint64_t(3);
    const uint32_t lead = uint32_t(dd.t0 - v0);
    const uint32_t nvec = (lead + dd.tlen + 3u) >> 2;
    for (uint32_t vi = threadIdx.x; vi < nvec; vi += 256) {
        const uint64_t e0 = v0 + uint64_t(vi) * 4u;
        const f32x4 a = load4<true>(sums + e0);
        f32x4 wq = load4<true>(op.w + e0), mq = load4<true>(op.m + e0), vq = {0.f, 0.f, 0.f, 0.f};
        if (OPT == kOptAdam) vq = load4<true>(op.v + e0);
        opt_apply<OPT>(a, wq, mq, vq, op, e0, int(vi * 4) - int(lead), int(dd.tlen));
    }
}

}  // namespace adacomp
