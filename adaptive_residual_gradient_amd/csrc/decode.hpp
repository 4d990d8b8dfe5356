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
};

__device__ __forceinline__ bool header_matches(const uint8_t* m, uint32_t nseg, uint32_t plan_hash) {
    return *reinterpret_cast<const uint32_t*>(m) == 0x43414441u &&
           *reinterpret_cast<const uint16_t*>(m + 4) == 1 &&
           *reinterpret_cast<const uint32_t*>(m + 8) == nseg &&
           *reinterpret_cast<const uint32_t*>(m + 12) == plan_hash;
}

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

// Per (chunk of decode tiles, message): survivors of each decode tile from
// the count words, offsets within the chunk, chunk totals.  Thread t takes
// tiles t, t + 256, t + 512, t + 768, so the lanes of a wavefront read
// neighbouring tiles' count words together; one block scan per round of
// 256 tiles gives the offsets in tile order.
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = uint32_t(i) * 256u + threadIdx.x;
        uint32_t s = 0;
        if (ok && t < n) {
            const uint32_t first_bin = (tb + t - sg.dt.tile_begin) * sg.dt.bpt;
            const uint32_t nb = min(sg.dt.bpt, sg.nbins - first_bin);
            const uint64_t a0 = sg.count_off + uint64_t(first_bin) * sg.wb;
            s = sum_count_words(m, a0, a0 + uint64_t(nb) * sg.wb, sg.wb);
        }
        cnt[i] = s;
    }
    uint32_t base = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = uint32_t(i) * 256u + threadIdx.x;
        uint32_t total;
        const uint32_t ex = block_exclusive_scan<256>(cnt[i], lw, &total);
        if (t < n) {
            ws.dcnt[uint64_t(k) * DT + tb + t] = cnt[i];
            ws.doff[uint64_t(k) * DT + tb + t] = base + ex;
        }
        base += total;
    }
    if (threadIdx.x == 0) ws.dchunk_cnt[uint64_t(k) * DC + c] = base;
}

// One block per message (at least one block): the message's validity,
// per-segment s and entry offsets, chunk bases.  Block 0 also counts the
// foreign messages into the status word.
__global__ void __launch_bounds__(256)
k_decode_base(MsgPtrs msgs, uint32_t K, const SegDev* __restrict__ segs, uint32_t nseg,
              uint32_t plan_hash, uint32_t DC, DecodeWs ws) {
    __shared__ uint32_t valid, bad;
    const uint32_t k = blockIdx.x;
    if (threadIdx.x == 0) {
        bad = 0;
        valid = 0;
        if (k < K) {
            valid = header_matches(msgs.p[k], nseg, plan_hash) ? 1u : 0u;
            ws.dvalid[k] = valid;
        }
    }
    __syncthreads();
    if (k == 0) {
        for (uint32_t j = threadIdx.x; j < K; j += 256)
            if (!header_matches(msgs.p[j], nseg, plan_hash)) atomicAdd(&bad, 1u);
    }
    if (k < K) {
        for (uint32_t l = threadIdx.x; l < nseg; l += 256) {
            const uint64_t i = uint64_t(k) * nseg + l;
            float s = 0.0f;
            uint64_t eoff = 0;
            if (valid) {
                const uint8_t* d = msgs.p[k] + 32 + 16 * uint64_t(l);
                s = *reinterpret_cast<const float*>(d);
                eoff = *reinterpret_cast<const uint64_t*>(d + 8);
            }
            ws.dseg_s[i] = s;
            ws.dseg_eoff[i] = eoff;
            const SegDev sg = segs[l];
            const uint64_t c0 = uint64_t(k) * DC + sg.dt.chunk_begin;
            uint32_t run = 0;
            // Chunk totals eight at a time, all requested before any is used.
            for (uint32_t c = 0; c < sg.dt.nchunks; c += 8) {
                uint32_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    v[u] = c + u < sg.dt.nchunks ? ws.dchunk_cnt[c0 + c + u] : 0u;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (c + u < sg.dt.nchunks) ws.dchunk_base[c0 + c + u] = run;
                    run += v[u];
                }
            }
        }
    }
    if (k == 0) {
        __syncthreads();
        if (threadIdx.x == 0) *ws.status = bad;
    }
}

// Index word at byte address a (w = 8 or 16 bits), read as the aligned
// 16-bit word that contains it; messages are 16-byte aligned and padded to a
// multiple of 16 bytes, so the read stays inside the message.
// The address is formed from integers kept in LDS, so it is cast to a
// global-address-space pointer (a global load, not a flat one).
typedef const __attribute__((address_space(1))) uint16_t* global_u16_ptr;

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
