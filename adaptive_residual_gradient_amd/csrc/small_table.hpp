// The end of the compress for small tables: scan, scale, message and encode
// in one kernel instead of three, and the one-launch variant.
//
// Method: "AdaComp (Adaptive Residual Gradient Compression)", AIMech curated
// page, definition paragraph and Mechanism claim on local-bin soft threshold
// and mean-g_max quantization (Algorithm 2); word widths from its Application
// claim (Table 2).
//
// For a small table each launch of the multi-kernel compress costs more than
// its work.  Once the tile pass has run, a table of at most a few thousand
// tiles fits in LDS: every workgroup of k_finish_small loads all the tiles'
// survivor counts and sums of bin maxima itself, forms the survivor offsets
// and each segment's s in LDS, and encodes its own share of the survivors;
// workgroup 0 also writes the directory, header and padding.  No workgroup
// waits for another, and the scattered stores of the encode are spread over
// the whole grid.
//
// The LDS work follows the multi-kernel path exactly where it rounds: the
// chunk sums of bin maxima use chunk_partial / wave_xor_sum / combine4 (one
// wavefront per chunk) and s comes from the same finalize_block, run on LDS
// arrays; every other result is an integer with one possible value.  So the
// bytes written equal the multi-kernel path's.
//
// k_compress_single puts the tile pass in the same launch: every workgroup
// runs one tile, publishes it and takes a ticket; the one that takes the last
// ticket runs the finish alone.  It is correct but slower on MI355X than tile
// pass + k_finish_small: the release of each tile (an L2 writeback per
// wavefront) and one CU's scattered stores outweigh the launch it saves.
// It is built for comparison, selected only by a plan flag.
#pragma once

#include "common.hpp"
#include "encode.hpp"
#include "tile_pass.hpp"

namespace adacomp {

struct SmallArgs {
    const SegDev* segs;
    const uint32_t* tile_seg;
    const uint32_t* tile_t0;        // flat index of each tile's first element (plan table)
    const uint32_t* vtiles0;        // single launch: tiles of shape 0, then of shape 1
    const uint32_t* vtiles1;
    const uint32_t* chunk_tile_begin;
    float* residue;
    const float* dW;
    uint8_t* msg;
    const uint32_t* stage;
    uint32_t* tile_cnt;
    double* tile_gsum;
    float* bin_max_out;             // single launch only
    uint64_t* sync;                 // single launch only
    uint64_t entries_begin;
    uint32_t n0;                    // single launch: tiles of shape 0
    uint32_t ntiles;
    uint32_t nchunks;
    uint32_t nseg;
    uint32_t plan_hash;
};

static_assert(uint64_t(ADACOMP_SMALL_TABLE_MAX_SPAN) <= (uint64_t(1) << 32),
              "small tables: flat element indices held in 32 bits");

// LDS tables of the finish (sizes in small_lds_bytes, layout.hpp).
struct SmallLds {
    double* tgs;       // [T] sums of bin maxima per tile
    double* cgs;       // [C] chunk sums of bin maxima
    uint64_t* seoff;   // [S] entry region offsets
    uint64_t* ssbase;  // [S + 1] survivors before each segment, then the total
    uint32_t* tpre;    // [T + 1] survivors before each tile (message order), then the total
    uint32_t* tt0;     // [T] flat index of each tile's first element
    uint32_t* tsi;     // [T] segment of each tile
    uint32_t* ccnt;    // [C] survivors per chunk
    uint32_t* cbase;   // [C] survivors before each chunk within its segment
    float* ss;         // [S] s
    uint32_t* sn;      // [S] survivors
    uint32_t* sltwb;   // [S] L_T << 2 | word bytes
    uint32_t* smag;    // [S] division magic
    uint32_t* ctb;     // [C + 1] first tile of each chunk, then T
};
__device__ __forceinline__ SmallLds small_lds(uint32_t* base, uint32_t T, uint32_t C, uint32_t S) {
    SmallLds t;
    t.tgs = reinterpret_cast<double*>(base);
    t.cgs = t.tgs + T;
    t.seoff = reinterpret_cast<uint64_t*>(t.cgs + C);
    t.ssbase = t.seoff + S;
    t.tpre = reinterpret_cast<uint32_t*>(t.ssbase + S + 1);
    t.tt0 = t.tpre + T + 1;
    t.tsi = t.tt0 + T;
    t.ccnt = t.tsi + T;
    t.cbase = t.ccnt + C;
    t.ss = reinterpret_cast<float*>(t.cbase + C);
    t.sn = reinterpret_cast<uint32_t*>(t.ss + S);
    t.sltwb = t.sn + S;
    t.smag = t.sltwb + S;
    t.ctb = t.smag + S;
    return t;
}

constexpr int kSmallBatch = 8;   // survivors per lane with their loads in flight together

// kSmallBatch x 64 survivors of one wavefront: their tiles and staged keys.
struct EncBatch {
    uint32_t key[kSmallBatch];
    uint32_t tile[kSmallBatch], e[kSmallBatch];
};

// Survivors base + 64u + lane (u < kSmallBatch) below e1, clamped to e1 - 1:
// find each one's tile in the LDS prefix and issue the load of its staged
// key (used by enc_store; needs only tpre and tt0).
__device__ __forceinline__ void enc_load(const SmallArgs& A, const SmallLds& L, uint32_t base,
                                         uint32_t e1, EncBatch& b) {
    const uint32_t lane = threadIdx.x & 63u, T = A.ntiles;
    uint32_t top = 1;   // largest power of two <= T
    while (top * 2u <= T) top *= 2u;
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u) {
        b.e[u] = min(base + 64u * u + lane, e1 - 1u);
        b.tile[u] = 0;
    }
    // The last tile t with tpre[t] <= e holds survivor e: a branch-free
    // search of fixed depth, the kSmallBatch searches advancing together.
    // A probe past the end reads tpre[T], the total, which exceeds every e.
    for (uint32_t step = top; step >= 1u; step >>= 1) {
#pragma unroll
        for (int u = 0; u < kSmallBatch; ++u) {
            const uint32_t c = b.tile[u] + step;
            b.tile[u] = L.tpre[min(c, T)] <= b.e[u] ? c : b.tile[u];
        }
    }
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u)
        b.key[u] = A.stage[L.tt0[b.tile[u]] + (b.e[u] - L.tpre[b.tile[u]])];
}

// Entry words and residue fix-up of a loaded batch (needs the finalized
// per-segment s and offsets).
__device__ __forceinline__ void enc_store(const SmallArgs& A, const SmallLds& L, uint32_t base,
                                          uint32_t e1, const EncBatch& b) {
    const uint32_t lane = threadIdx.x & 63u;
    // G of every survivor of the batch (the tile pass left residue = G there).
    float gq[kSmallBatch];
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u)
        gq[u] = A.residue[uint64_t(L.tt0[b.tile[u]]) + (b.key[u] & 0x7FFFFFFFu)];
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u) {
        if (base + 64u * u + lane < e1) {
            const uint32_t t = b.tile[u], si = L.tsi[t];
            const uint32_t lt = L.sltwb[si] >> 2, wb = L.sltwb[si] & 3u;
            const uint32_t x = b.key[u] & 0x7FFFFFFFu, neg = b.key[u] >> 31;
            const uint32_t bin = div_bin(x, lt, L.smag[si]);
            const uint32_t topbit = wb == 1u ? 7u : 15u;
            put_word(A.msg + L.seoff[si] + uint64_t(b.e[u] - uint32_t(L.ssbase[si])) * wb, wb,
                     (neg << topbit) | (x - bin * lt));
            const float gv = gq[u], sv = L.ss[si];
            // residue <- G - G_q with G_q = sign(G) * s
            A.residue[uint64_t(L.tt0[t]) + x] = neg ? gv + sv : gv - sv;
        }
    }
}

// The finish by one block of 256 threads after every tile is done: LDS
// tables, survivor offsets per tile, s, entry offsets and survivors per
// segment (write_msg: also the directory, header and padding), then the
// entry words and residue fix-ups of wavefront w of W's share of the
// survivors, [S*w/W, S*(w+1)/W).  The first batch of staged keys is loaded
// before the finalize step, so the two memory round trips overlap.
__device__ __forceinline__ void small_finish(const SmallArgs& A, uint32_t* dyn, uint32_t* lw,
                                             uint64_t* lsz, uint64_t* lns, uint32_t* nlong,
                                             bool write_msg, uint64_t w, uint64_t W) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
    const uint32_t T = A.ntiles, C = A.nchunks, S = A.nseg;
    const SmallLds L = small_lds(dyn, T, C, S);
    if (tid == 0) *nlong = 0;

    // Every table in one pass of independent loads.
    for (uint32_t t = tid; t < T; t += 256) {
        L.tpre[t] = A.tile_cnt[t];   // counts, turned into a prefix below
        L.tgs[t] = A.tile_gsum[t];
        L.tsi[t] = A.tile_seg[t];
        L.tt0[t] = A.tile_t0[t];
    }
    for (uint32_t c = tid; c <= C; c += 256) L.ctb[c] = A.chunk_tile_begin[c];
    for (uint32_t l = tid; l < S; l += 256) {
        L.sltwb[l] = (A.segs[l].lt << 2) | A.segs[l].wb;
        L.smag[l] = A.segs[l].magic;
    }
    __syncthreads();
    // Chunk sums of bin maxima in the fixed order: one thread per chunk of
    // at most 32 tiles, one wavefront per longer chunk (listed in cbase,
    // which finalize fills only later).
    for (uint32_t c = tid; c < C; c += 256) {
        const uint32_t tb = L.ctb[c], n = L.ctb[c + 1] - tb;
        if (n <= kShortChunkTiles) L.cgs[c] = chunk_sum_short(L.tgs, tb, n);
        else L.cbase[atomicAdd(nlong, 1u)] = c;
    }
    __syncthreads();
    for (uint32_t i = wv; i < *nlong; i += 4) {
        const uint32_t c = L.cbase[i], tb = L.ctb[c], n = L.ctb[c + 1] - tb;
        double q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = wave_xor_sum(chunk_partial(L.tgs, tb, n, 64u * k + lane));
        if (lane == 0) L.cgs[c] = combine4(q[0], q[1], q[2], q[3]);
    }
    // Survivors before each tile, in tile order (= message order).
    {
        const uint32_t a = uint32_t(uint64_t(T) * tid / 256u), b = uint32_t(uint64_t(T) * (tid + 1) / 256u);
        uint32_t mine = 0;
        for (uint32_t t = a; t < b; ++t) mine += L.tpre[t];
        uint32_t total;
        uint32_t run = block_exclusive_scan<256>(mine, lw, &total);
        for (uint32_t t = a; t < b; ++t) {
            const uint32_t c = L.tpre[t];
            L.tpre[t] = run;
            run += c;
        }
        if (tid == 0) L.tpre[T] = total;
    }
    __syncthreads();
    for (uint32_t c = tid; c < C; c += 256) L.ccnt[c] = L.tpre[L.ctb[c + 1]] - L.tpre[L.ctb[c]];

    const uint64_t total = L.tpre[T];
    const uint32_t e0 = uint32_t(total * w / W), e1 = uint32_t(total * (w + 1) / W);
    EncBatch b;
    if (e0 < e1) enc_load(A, L, e0, e1, b);   // wavefront-uniform
    __syncthreads();
    // s, entry regions (and the message's directory and header): the
    // multi-kernel path's finalize.
    finalize_block(A.segs, S, A.plan_hash, A.entries_begin, L.ccnt, L.cgs, L.cbase, L.ss, L.sn,
                   L.seoff, L.ssbase, A.msg, lsz, lns, write_msg);
    __syncthreads();
    if (e0 >= e1) return;   // wavefront-uniform; no barrier follows
    enc_store(A, L, e0, e1, b);
    for (uint32_t base = e0 + 64u * kSmallBatch; base < e1; base += 64u * kSmallBatch) {
        enc_load(A, L, base, e1, b);
        enc_store(A, L, base, e1, b);
    }
}

// After the tile pass: every workgroup runs the finish on its own tables;
// wavefront w of the grid's W encodes its share.
__global__ void __launch_bounds__(256) k_finish_small(SmallArgs A) {
    extern __shared__ uint64_t dyn64[];   // 8-byte aligned: doubles live there
    __shared__ uint32_t lw[4], nlong;
    __shared__ uint64_t lsz[4], lns[4];
    small_finish(A, reinterpret_cast<uint32_t*>(dyn64), lw, lsz, lns, &nlong, blockIdx.x == 0,
                 uint64_t(blockIdx.x) * 4u + (threadIdx.x >> 6), uint64_t(gridDim.x) * 4u);
}

// ---------------------------------------------------------------------------
// One launch: the tile pass, then the finish by the last workgroup.
//
// The ticket counter is one 64-bit word at the start of the compress
// workspace: a 48-bit tag above a 16-bit count.  A word holding the tag
// counts tickets; any other content is claimed by the first workgroup to
// arrive (compare-and-swap to tag | 1), so the workspace needs no clearing.
// The last workgroup puts back tag | 0 for the next call.  Only a word that
// already holds the tag with a nonzero count (which a call stopped part way
// leaves behind) would miscount.
// ---------------------------------------------------------------------------
constexpr uint64_t kSyncTag = 0xFFF1ADAC0DE5ull;   // top 32 bits of the word: a float NaN pattern
constexpr uint64_t kSyncIdle = kSyncTag << 16;

// Ticket of the calling workgroup, 0-based (one thread per workgroup).
__device__ __forceinline__ uint32_t sync_ticket(uint64_t* word) {
    uint64_t cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // At most two rounds: a failed claim means another workgroup has just
    // written the tag.  The bound only guards against a foreign writer.
    for (int round = 0; round < 4; ++round) {
        if ((cur >> 16) == kSyncTag)
            return uint32_t(__hip_atomic_fetch_add(word, 1ull, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) & 0xFFFFu);
        if (__hip_atomic_compare_exchange_strong(word, &cur, kSyncIdle | 1ull, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return 0u;
    }
    return kSentinel;   // never the last ticket
}

static_assert(kVarThreads[0] == 256 && kVarThreads[1] == 256, "single launch: 256-thread tiles");

__global__ void __launch_bounds__(256) k_compress_single(SmallArgs A) {
    constexpr int NCH = 4 * (kVarVecs[0] > kVarVecs[1] ? kVarVecs[0] : kVarVecs[1]);
    extern __shared__ uint64_t dyn64[];   // 8-byte aligned: the finish keeps doubles there
    uint32_t* dyn = reinterpret_cast<uint32_t*>(dyn64);
    __shared__ uint32_t ch_tot[NCH];
    __shared__ uint32_t lw[4], nlong;
    __shared__ uint64_t lsz[4], lns[4];
    __shared__ uint32_t last;

    // Small tables keep their residue stores cached (see kCachedResidueMaxElems).
    static_assert(ADACOMP_SMALL_TABLE_MAX_SPAN <= kCachedResidueMaxElems, "small tables are cached");
    if (blockIdx.x < A.n0) {
        TileRegs<kVarVecs[0]> t;
        load_tile<256, kVarVecs[0]>(t, A.segs, A.tile_seg, A.vtiles0, blockIdx.x, A.residue, A.dW);
        process_tile<256, kVarVecs[0], false>(t, dyn, A.segs, A.tile_seg, A.residue, A.msg,
                                              const_cast<uint32_t*>(A.stage), A.tile_cnt,
                                              A.tile_gsum, A.bin_max_out, ch_tot);
    } else {
        TileRegs<kVarVecs[1]> t;
        load_tile<256, kVarVecs[1]>(t, A.segs, A.tile_seg, A.vtiles1, blockIdx.x - A.n0,
                                    A.residue, A.dW);
        process_tile<256, kVarVecs[1], false>(t, dyn, A.segs, A.tile_seg, A.residue, A.msg,
                                              const_cast<uint32_t*>(A.stage), A.tile_cnt,
                                              A.tile_gsum, A.bin_max_out, ch_tot);
    }
    // Publish: every wavefront releases its own stores at agent scope (a
    // workgroup barrier alone does not wait for them to leave the CU), the
    // barrier orders those releases before the ticket, and the last
    // workgroup acquires.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
        const bool is_last = sync_ticket(A.sync) == A.ntiles - 1u;
        if (is_last) {
            __hip_atomic_store(A.sync, kSyncIdle, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        last = is_last ? 1u : 0u;
    }
    __syncthreads();
    if (last == 0u) return;   // workgroup-uniform
    small_finish(A, dyn, lw, lsz, lns, &nlong, true, threadIdx.x >> 6, 4u);
}

}  // namespace adacomp
