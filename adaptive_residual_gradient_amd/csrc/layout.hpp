// Host-side plan layout for the AdaComp library: validation of a segment
// table, work tiles, message layout and workspace layout.  No HIP calls here.
//
// Work decomposition.  Each segment (one layer) is cut into tiles of whole
// bins, so that every bin maximum, survivor count and compaction is local to
// one workgroup and no cross-workgroup combination is needed for a bin.
//   - narrow tiles: 256 threads x 2 float4 per thread per array, at most 2048
//     elements (four bins of 500, forty bins of 50), for L_T <= 2045;
//   - medium tiles: 256 threads x 4 float4, at most 4096 elements, for
//     L_T <= 4093;
//   - long bins (L_T > 4093): one bin per tile, streamed in chunks.
// Bins per tile are chosen so that tile starts fall on 16-byte boundaries
// whenever that fits, which keeps every load and store a whole float4 except
// at the ends of segments.
#pragma once

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "../../include/adacomp.h"

#if defined(__HIPCC__)
#define ADACOMP_HD __host__ __device__
#else
#define ADACOMP_HD
#endif

namespace adacomp {

// Tile shapes.  Shapes 0 and 1 hold a tile of whole bins in registers
// (threads per workgroup x float4 per thread per array); a layer uses the
// first of them whose capacity holds one bin plus the up-to-3 leading
// elements of an unaligned tile start.  Longer bins take shape 2: one bin
// per tile, streamed twice by 256 threads in chunks of 256 x 2 float4.
// Shape 0 at 2 float4 per thread is the fastest for L_T = 500 (3 or 4:
// 2.07 and 2.11 ms against 1.97-2.01 ms on the 1.07e9-element workload;
// 512- or 1024-thread tiles: 2.4-2.6 ms).
constexpr int kVariants = 3;
constexpr uint32_t kVarThreads[kVariants] = {256, 256, 256};
constexpr uint32_t kVarVecs[kVariants] = {2, 4, 2};   // shape 2: per chunk
constexpr uint32_t kLongCap = ADACOMP_MAX_BIN_LEN + 4;   // one bin and an unaligned start
// Long bins that span at most this many chunks of shape 2 are held in
// registers for both passes (4 chunks of 256 x 2 float4: L_T up to 8189).
constexpr int kLongRegChunks = 4;
constexpr uint32_t var_cap(int v) { return v == 2 ? kLongCap : kVarThreads[v] * kVarVecs[v] * 4; }
constexpr uint32_t kMaxCap = 1024 * 9 * 4;   // 36864 elements: long-bin decode tiles
constexpr uint32_t kChunkTiles = 1024;  // tiles per scan chunk (4 per thread of a 256-thread block)
// Decode tiles per count chunk (k_decode_count: one workgroup per chunk and
// message) on tables of fewer than kDecSmallTableTiles decode tiles: a tile
// per thread, so that the count words of a layer are read by four times the
// workgroups.  Larger tables keep kChunkTiles (the launch count there
// already fills the chip).  Measured on MI355X, K = 16: conv stack 35.2 ->
// 31.0 us, ResNet-50 115.6 -> 110.9 us, FC/LSTM 57.8 -> 56.0 us; the
// 1.07e9-element table 1.166 -> 1.18 ms with 256.
constexpr uint32_t kDecChunkTiles = 256;
constexpr uint64_t kDecSmallTableTiles = 65536;
// Tables of at most this many elements write the residue in the tile pass with
// ordinary (cached) stores, larger ones non-temporally.  The finish rewrites
// the residue at every sent element; while the whole residue (here at most
// 256 MB) can stay in the 256 MB Infinity Cache those partial-line stores hit
// it.  Compress calls measured with each hint, 16.7 M-element layers at
// L_T 50 / 500 (us): 16 M 72 / 65 cached against 81 / 72 non-temporal;
// 32 M 120 / 105 against 140 / 122; 64 M 247 / 191 against 262 / 221;
// 128 M 598 / 500 against 557 / 450 (there the cached stores evict data the
// stream still needs).
constexpr uint64_t kCachedResidueMaxElems = uint64_t(1) << 26;
constexpr uint32_t kPrefWords = 8192;   // LDS words for per-message bin prefixes in decode
constexpr uint64_t kAlign = 256;        // workspace sub-buffer alignment

// How one layer is cut into tiles of whole bins.
struct TileSpec {
    uint32_t bpt;         // bins per tile
    uint32_t tile_begin;  // first global tile of the layer
    uint32_t ntiles;
    uint32_t chunk_begin; // first scan chunk (kChunkTiles tiles each) of the layer
    uint32_t nchunks;
    uint32_t variant;     // tile shape index
};

// Per-segment parameters read by every kernel (112 bytes).
struct SegDev {
    uint64_t off;        // element offset in the flat buffers
    uint64_t numel;
    uint64_t bin_base;   // global index of the segment's first bin
    uint64_t count_off;  // byte offset of the segment's count region in a message
    uint32_t lt;         // bin length L_T
    uint32_t magic;      // floor(2^32 / lt) + 1: exact x / lt for x < 2^16 (lt >= 2)
    uint32_t nbins;
    uint32_t wb;         // index word bytes: 1 if lt < 64 else 2
    TileSpec ct;         // compress tiles
    TileSpec dt;         // decode tiles
    uint32_t flags;      // 0 or ADACOMP_SEG_LS
    uint32_t pad[3];
};
static_assert(sizeof(SegDev) == 112, "SegDev layout");

// Exact x / lt for 0 <= x < 2^16 and 2 <= lt <= 2^16 with magic =
// floor(2^32 / lt) + 1: the product overshoots x / lt by x * e / 2^32 with
// 0 < e <= 1, which stays below 2^-16 <= 1/lt, so the floor is unchanged.
ADACOMP_HD inline uint32_t div_bin(uint32_t x, uint32_t lt, uint32_t magic) {
    return lt == 1u ? x : static_cast<uint32_t>((uint64_t(x) * magic) >> 32);
}

// Geometry of one tile: its bins, elements and the float4 it touches.
struct TileGeom {
    uint32_t first_bin;  // first bin of the tile within its segment
    uint32_t nb;         // bins in the tile
    uint32_t tlen;       // elements in the tile
    uint32_t lead;       // t0 - v0 (0..3)
    uint32_t nvec;       // float4 the tile touches
    uint64_t t0;         // flat index of the tile's first element
    uint64_t v0;         // t0 rounded down to a multiple of 4
};

ADACOMP_HD inline TileGeom tile_geom(const SegDev& sg, const TileSpec& ts, uint32_t tile) {
    TileGeom g;
    const uint32_t local = tile - ts.tile_begin;
    g.first_bin = local * ts.bpt;
    const uint32_t left = sg.nbins - g.first_bin;
    g.nb = ts.bpt < left ? ts.bpt : left;
    const uint64_t e0 = uint64_t(g.first_bin) * sg.lt;
    const uint64_t rest = sg.numel - e0;
    const uint64_t want = uint64_t(g.nb) * sg.lt;
    g.tlen = static_cast<uint32_t>(want < rest ? want : rest);
    g.t0 = sg.off + e0;
    g.v0 = g.t0 & ~uint64_t(3);
    g.lead = static_cast<uint32_t>(g.t0 - g.v0);
    g.nvec = (g.lead + g.tlen + 3u) >> 2;
    return g;
}

// The tiles of one kind over the whole table.
struct Tiling {
    std::vector<uint32_t> tile_seg;          // [T] segment of each tile
    std::vector<uint32_t> by_variant[3];     // tile ids of each shape, in order
    std::vector<uint32_t> chunk_tile_begin;  // [C + 1]
    std::vector<uint32_t> chunk_seg;         // [C]
    uint32_t max_bpt[3] = {0, 0, 0};
    uint32_t max_span_vecs[3] = {0, 0, 0};   // most float4 one tile touches
    uint64_t ntiles = 0, nchunks = 0;
    uint32_t chunk_tiles = kChunkTiles;      // tiles per chunk (at most kChunkTiles)
};

// Everything the decode apply kernel needs about one decode tile, built at
// plan time in launch order so that a workgroup starts with a single load.
// What k_decode_count needs of one decode count chunk, read with one load
// (instead of the chunk's layer index and then the layer's record).
struct CountChunk {
    uint64_t count_off;   // message byte offset of the layer's first count word
    uint64_t numel;       // elements of the layer
    uint32_t tile0;       // global index of the chunk's first decode tile
    uint32_t ntiles;      // decode tiles in the chunk
    uint32_t first_bin;   // the layer's bin index of the chunk's first bin
    uint32_t bpt;         // bins per decode tile
    uint32_t nbins;       // bins of the layer
    uint32_t wb;          // bytes per word
    uint32_t lt;          // bin length
    uint32_t pad;
};
static_assert(sizeof(CountChunk) == 48, "CountChunk layout");

struct DecDesc {
    uint64_t t0;        // flat index of the tile's first element
    uint64_t count_at;  // message byte offset of the tile's first count word
    uint32_t tile;      // global decode tile index
    uint32_t si;        // segment
    uint32_t nb;        // bins in the tile
    uint32_t tlen;      // elements in the tile
    uint32_t lt;
    uint32_t wb;
    uint32_t chunk;     // global decode scan chunk
    uint32_t pad;
};
static_assert(sizeof(DecDesc) == 48, "DecDesc layout");

// Decode tiles: accumulated in LDS up to kDecCap elements (L_T <= 4093),
// otherwise one bin per tile accumulated in place in out.
constexpr uint32_t kDecCap = 4096;
constexpr int kDecVariants = 2;
constexpr uint32_t kDecThreads[kDecVariants] = {256, 1024};

// Dynamic LDS bytes of the decode apply kernel: the tile accumulator
// (acc_words floats, rounded to even), per message a u64 message address
// (0 for a foreign message), per group message a u64 entry address, per
// message s, the per-wavefront flat prefixes and the bin prefixes of KG
// messages.
inline uint32_t decode_lds_bytes(uint32_t acc_words, uint32_t K, uint32_t KG, uint32_t pstride,
                                 uint32_t nw) {
    const uint32_t accw = (acc_words + 1u) & ~1u;
    return 4u * (accw + 2u * K + 2u * KG + K + nw * (KG + 1u) + KG * pstride);
}

// Messages per decode group: at most 64 (one wavefront lane each) and as many
// bin prefixes as fit in kPrefWords.
inline uint32_t decode_group(uint32_t K, uint32_t pstride) {
    uint32_t kg = kPrefWords / pstride;
    if (kg > 64u) kg = 64u;
    if (kg > K) kg = K;
    return kg < 1u ? 1u : kg;
}

// The LDS decode tiles (k_decode_tiles) hold one 32-bit word per element for
// a group of up to kMaskMsgs messages: a hit bit and a sign bit per message.
constexpr uint32_t kMaskMsgs = 16;
// Entry blocks (16 bytes) per tile that k_decode_tiles_sum copies straight
// into LDS together with the count words.
constexpr uint32_t kPreBlocks = 128;

// Launch position of workgroup b of n, in runs of kXcdGroup consecutive
// positions per XCD.  The dispatcher hands workgroups to the 8 XCDs in turn
// (workgroup b to XCD b % 8), and each XCD has its own L2.  Neighbouring
// decode tiles share the cache lines of their per-message count words,
// entry words and entry records, so with consecutive positions on different
// XCDs each such line is fetched into several L2s.  Workgroup b takes
// position 8G*floor(b/8G) + G*(b % 8) + floor(b/8) % G (G = kXcdGroup), and
// the last n mod 8G workgroups keep their own positions: a bijection of
// [0, n).  Runs of 8 made the plain K = 16 decode of 1.07e9 elements
// (k_decode_tiles_sum) 1.096 -> 1.073 ms; in k_decode_tiles they made the
// fused SGD and Adam steps slower (2.79 -> 2.91 ms, 4.28 -> 4.36 ms), and
// one contiguous run per XCD slowed every decode (SGD 3.21 ms).
constexpr uint32_t kXcdGroup = 8;
ADACOMP_HD constexpr uint32_t xcd_grouped(uint32_t b, uint32_t n) {
    return b >= n / (8u * kXcdGroup) * (8u * kXcdGroup)
               ? b
               : (b & ~(8u * kXcdGroup - 1u)) | ((b & 7u) * kXcdGroup) | ((b >> 3) & (kXcdGroup - 1u));
}

// Dynamic LDS bytes of k_decode_tiles: acc_words mask words (and as many sum
// words with SEP), per message its address, per group message its first
// entry's address, entry count and s, and the group's bin prefixes.
// k_decode_tiles can keep, for a group whose runs hold at most 4 tblw entry
// words, the start of each bin (one byte, tiles of at most 128 bins) in the
// place of the bin prefixes (tblw words, at least the prefixes' own).
constexpr uint32_t kTblBytes = 10240;
// LDS words of k_decode_tiles' bin prefixes (16 bits each).
inline uint32_t decode_tiles_pref_words(uint32_t KG, uint32_t pstride) { return (KG * pstride + 1u) / 2u; }
inline uint32_t decode_tiles_lds_bytes(uint32_t acc_words, uint32_t K, uint32_t KG,
                                       uint32_t pstride, bool sep, uint32_t tblw) {
    const uint32_t accw = (acc_words + 3u) & ~3u;
    const uint32_t pw = decode_tiles_pref_words(KG, pstride) > tblw ? decode_tiles_pref_words(KG, pstride) : tblw;
    return 4u * (accw * (sep ? 2u : 1u) + 2u * K + 2u * KG + 2u * KG + pw);
}

// Dynamic LDS bytes of k_decode_tiles_sum (K <= kMaskMsgs messages): the mask
// words, kPreBlocks entry blocks and a word of placement data each, per
// message its address, entry record and s, and the bin prefixes.
inline uint32_t decode_sum_lds_bytes(uint32_t acc_words, uint32_t K, uint32_t pstride) {
    const uint32_t accw = (acc_words + 3u) & ~3u;
    return 4u * (accw + 5u * kPreBlocks + 5u * K + K * pstride);
}

// Messages per group of k_decode_tiles: at most kMaskMsgs, and as many bin
// prefixes as fit in kTilesPrefWords LDS words (at least one message).
constexpr uint32_t kTilesPrefWords = 4096;
inline uint32_t decode_tiles_group(uint32_t K, uint32_t pstride) {
    uint32_t kg = kTilesPrefWords / pstride;
    if (kg > kMaskMsgs) kg = kMaskMsgs;
    if (kg > K) kg = K;
    return kg < 1u ? 1u : kg;
}

struct Layout {
    uint32_t nseg = 0;
    uint32_t plan_hash = 0;
    std::vector<SegDev> segs;
    Tiling ct;                               // compress tiles
    Tiling dt;                               // decode tiles
    uint64_t total_numel = 0, total_bins = 0;
    bool has_ls = false;   // some segment uses hard local selection
    uint64_t span = 0;   // max(offset + numel) rounded up to 4: the flat buffers' minimum length
    uint64_t counts_begin = 0, entries_begin = 0, capacity = 0;

    // Compress workspace (byte offsets).  ws_sync: the single-launch path's
    // ticket word, in a slot of its own that no other kernel writes.
    uint64_t ws_sync = 0;
    uint64_t ws_stage = 0, ws_tile_cnt = 0, ws_tile_gsum = 0, ws_tile_off = 0;
    uint64_t ws_chunk_cnt = 0, ws_chunk_gsum = 0, ws_chunk_base = 0;
    uint64_t ws_seg_s = 0, ws_seg_nsurv = 0, ws_seg_eoff = 0, ws_seg_sbase = 0, ws_compress = 0;

    // Decode workspace: fixed part, then per-message arrays.
    uint64_t dws_fixed = 0, dws_per_msg = 0;
};

inline uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// FNV-1a, 32 bit, over each segment's offset, numel (8 bytes each), bin_len
// and flags (4 bytes each), little-endian, in table order.
inline uint32_t table_hash(const adacomp_segment* s, uint32_t n) {
    uint32_t h = 0x811C9DC5u;
    auto mix = [&h](uint64_t v, int bytes) {
        for (int i = 0; i < bytes; ++i) {
            h ^= static_cast<uint32_t>((v >> (8 * i)) & 0xFFu);
            h *= 0x01000193u;
        }
    };
    for (uint32_t i = 0; i < n; ++i) {
        mix(s[i].offset, 8);
        mix(s[i].numel, 8);
        mix(s[i].bin_len, 4);
        mix(s[i].flags, 4);
    }
    return h;
}

// Bins per tile for bin length lt and tile capacity cap (elements): as many
// whole bins as fit, rounded so that tiles start 16-byte aligned if possible;
// otherwise leave room for the up-to-3-element lead of an unaligned start.
inline uint32_t bins_per_tile(uint32_t lt, uint32_t cap, uint32_t nbins) {
    uint32_t bpt = cap / lt;
    if (bpt >= nbins) return nbins;   // one tile holds the segment; it starts aligned
    const uint32_t a = 4u / std::gcd(lt, 4u);
    if ((static_cast<uint64_t>(bpt) * lt) % 4 != 0) {
        const uint32_t aligned = bpt / a * a;
        bpt = aligned >= 1 ? aligned : (cap - 3) / lt;
    }
    return bpt;
}

inline int build_layout(const adacomp_segment* segs, uint32_t nseg, Layout& L) {
    if (segs == nullptr || nseg == 0) return ADACOMP_ERR_INVALID_ARGUMENT;
    for (uint32_t i = 0; i < nseg; ++i) {
        const adacomp_segment& s = segs[i];
        if (s.numel == 0 || (s.flags != 0 && s.flags != ADACOMP_SEG_LS)) return ADACOMP_ERR_INVALID_ARGUMENT;
        if (s.bin_len == 0 || s.bin_len > ADACOMP_MAX_BIN_LEN) return ADACOMP_ERR_UNSUPPORTED_BIN;
        if (s.offset % 4 != 0) return ADACOMP_ERR_MISALIGNED;
        if (s.numel >= (uint64_t(1) << 32)) return ADACOMP_ERR_TOO_LARGE;
        if (s.offset > (uint64_t(1) << 48)) return ADACOMP_ERR_TOO_LARGE;
    }
    {   // overlap check on the table sorted by offset
        std::vector<uint32_t> ord(nseg);
        std::iota(ord.begin(), ord.end(), 0u);
        std::sort(ord.begin(), ord.end(),
                  [&](uint32_t a, uint32_t b) { return segs[a].offset < segs[b].offset; });
        for (uint32_t i = 1; i < nseg; ++i) {
            const adacomp_segment& p = segs[ord[i - 1]];
            if (p.offset + p.numel > segs[ord[i]].offset) return ADACOMP_ERR_OVERLAP;
        }
    }

    L = Layout();
    {   // the decode tiles the cut below makes, for the chunk size
        uint64_t dtiles = 0;
        for (uint32_t i = 0; i < nseg; ++i) {
            const uint32_t nbins = static_cast<uint32_t>((segs[i].numel + segs[i].bin_len - 1) / segs[i].bin_len);
            const uint32_t cap = segs[i].bin_len + 3 <= kDecCap ? kDecCap : kMaxCap;
            const uint32_t bpt = bins_per_tile(segs[i].bin_len, cap, nbins);
            dtiles += (nbins + bpt - 1) / bpt;
        }
        L.dt.chunk_tiles = dtiles < kDecSmallTableTiles ? kDecChunkTiles : kChunkTiles;
    }
    L.nseg = nseg;
    L.plan_hash = table_hash(segs, nseg);
    L.segs.resize(nseg);
    L.counts_begin = round_up(32 + 16 * uint64_t(nseg), 16);
    uint64_t count_at = L.counts_begin;
    uint64_t bins = 0;
    // Cut layer i into tiles of spec ts (shape v, capacity cap elements).
    auto cut = [&](Tiling& T, TileSpec& ts, uint32_t i, uint32_t v, uint32_t cap,
                   uint32_t max_bins) -> int {
        const SegDev& d = L.segs[i];
        ts.variant = v;
        ts.bpt = std::min(bins_per_tile(d.lt, cap, d.nbins), max_bins);
        ts.ntiles = (d.nbins + ts.bpt - 1) / ts.bpt;
        if (T.ntiles + ts.ntiles >= (uint64_t(1) << 31)) return ADACOMP_ERR_TOO_LARGE;
        ts.tile_begin = static_cast<uint32_t>(T.ntiles);
        ts.nchunks = (ts.ntiles + T.chunk_tiles - 1) / T.chunk_tiles;
        ts.chunk_begin = static_cast<uint32_t>(T.nchunks);
        // Most float4 any tile touches: an unaligned start adds up to 3
        // leading elements.
        const uint64_t tile_elems = std::min<uint64_t>(uint64_t(ts.bpt) * d.lt, d.numel);
        const bool aligned = (uint64_t(ts.bpt) * d.lt) % 4 == 0 || ts.ntiles == 1;
        const uint64_t vecs = (tile_elems + (aligned ? 0 : 3) + 3) / 4;
        if (vecs * 4 > cap) return ADACOMP_ERR_UNSUPPORTED_BIN;
        T.max_span_vecs[v] = std::max<uint32_t>(T.max_span_vecs[v], uint32_t(vecs));
        T.max_bpt[v] = std::max(T.max_bpt[v], ts.bpt);
        for (uint32_t t = 0; t < ts.ntiles; ++t) {
            T.tile_seg.push_back(i);
            T.by_variant[v].push_back(static_cast<uint32_t>(T.ntiles + t));
        }
        for (uint32_t c = 0; c < ts.nchunks; ++c) {
            T.chunk_tile_begin.push_back(static_cast<uint32_t>(T.ntiles + uint64_t(c) * T.chunk_tiles));
            T.chunk_seg.push_back(i);
        }
        T.ntiles += ts.ntiles;
        T.nchunks += ts.nchunks;
        return ADACOMP_OK;
    };
    for (uint32_t i = 0; i < nseg; ++i) {
        const adacomp_segment& s = segs[i];
        SegDev& d = L.segs[i];
        d = SegDev{};
        d.off = s.offset;
        d.numel = s.numel;
        d.lt = s.bin_len;
        d.magic = s.bin_len >= 2 ? static_cast<uint32_t>((uint64_t(1) << 32) / s.bin_len + 1) : 0u;
        const uint64_t nb = (s.numel + s.bin_len - 1) / s.bin_len;
        d.nbins = static_cast<uint32_t>(nb);
        d.wb = s.bin_len < 64 ? 1u : 2u;
        d.flags = s.flags;
        L.has_ls |= s.flags == ADACOMP_SEG_LS;
        d.bin_base = bins;
        d.count_off = count_at;
        uint32_t cv = kVariants - 1;
        for (int v = kVariants - 1; v >= 0; --v)
            if (s.bin_len + 3 <= var_cap(v)) cv = uint32_t(v);
        int st = cut(L.ct, d.ct, i, cv, var_cap(int(cv)), cv == 2 ? 1u : ~0u);
        if (st != ADACOMP_OK) return st;
        const uint32_t dv = s.bin_len + 3 <= kDecCap ? 0u : 1u;
        st = cut(L.dt, d.dt, i, dv, dv == 0 ? kDecCap : kMaxCap, ~0u);
        if (st != ADACOMP_OK) return st;
        bins += nb;
        count_at = round_up(count_at + nb * d.wb, 16);
        L.total_numel += s.numel;
        L.span = std::max<uint64_t>(L.span, round_up(s.offset + s.numel, 4));
    }
    L.ct.chunk_tile_begin.push_back(static_cast<uint32_t>(L.ct.ntiles));
    L.dt.chunk_tile_begin.push_back(static_cast<uint32_t>(L.dt.ntiles));
    L.total_bins = bins;
    L.entries_begin = count_at;
    uint64_t cap = count_at;
    for (uint32_t i = 0; i < nseg; ++i) cap = round_up(cap + L.segs[i].numel * L.segs[i].wb, 16);
    L.capacity = cap;
    const uint64_t tiles = L.ct.ntiles, chunks = L.ct.nchunks;

    // Compress workspace.
    uint64_t w = 0;
    auto take = [&w](uint64_t bytes) {
        const uint64_t at = w;
        w = round_up(w + bytes, kAlign);
        return at;
    };
    L.ws_sync = take(8);
    L.ws_stage = take(4 * L.span);     // per tile at its offset: survivor keys (sign | offset), then G where it fits
    L.ws_tile_cnt = take(4 * tiles);
    L.ws_tile_gsum = take(8 * tiles);
    L.ws_tile_off = take(4 * tiles);
    L.ws_chunk_cnt = take(4 * chunks);
    L.ws_chunk_gsum = take(8 * chunks);
    L.ws_chunk_base = take(4 * chunks);
    L.ws_seg_s = take(4 * uint64_t(nseg));
    L.ws_seg_nsurv = take(4 * uint64_t(nseg));
    L.ws_seg_eoff = take(8 * uint64_t(nseg));
    L.ws_seg_sbase = take(8 * (uint64_t(nseg) + 1));   // survivors before each segment, then the total
    L.ws_compress = w;

    // Decode workspace for K messages: a status block, then arrays indexed by
    // message: decode-tile counts and offsets [K*DT], chunk counts and bases
    // [K*DC], per-segment s and entry offsets [K*nseg], per-message validity
    // [K], and an 8-byte entry record per LDS decode tile [K*P], P <= DT.
    // Each array is kAlign-aligned, so fixed covers the padding of all.
    L.dws_fixed = 10 * kAlign;
    L.dws_per_msg = round_up(16 * L.dt.ntiles + 8 * L.dt.nchunks + 12 * uint64_t(nseg) + 4, 16);
    return ADACOMP_OK;
}

// Descriptors of the decode tiles of shape v, in launch order.
inline std::vector<DecDesc> decode_descs(const Layout& L, int v) {
    std::vector<DecDesc> out;
    out.reserve(L.dt.by_variant[v].size());
    for (uint32_t tile : L.dt.by_variant[v]) {
        const uint32_t si = L.dt.tile_seg[tile];
        const SegDev& sg = L.segs[si];
        const TileGeom g = tile_geom(sg, sg.dt, tile);
        DecDesc d{};
        d.t0 = g.t0;
        d.count_at = sg.count_off + uint64_t(g.first_bin) * sg.wb;
        d.tile = tile;
        d.si = si;
        d.nb = g.nb;
        d.tlen = g.tlen;
        d.lt = sg.lt;
        d.wb = sg.wb;
        d.chunk = sg.dt.chunk_begin + (tile - sg.dt.tile_begin) / L.dt.chunk_tiles;
        out.push_back(d);
    }
    return out;
}

// LDS bytes of the small-table finish for T tiles, C scan chunks and S
// segments: per tile a double and three words (plus one total), per chunk a
// double and three words (plus one), per segment two 64-bit and four 32-bit
// words (plus one 64-bit total).
ADACOMP_HD constexpr uint64_t small_lds_bytes(uint64_t T, uint64_t C, uint64_t S) {
    return 8 * T + 4 * (T + 1) + 8 * T + 8 * C + 4 * (C + 1) + 8 * C + 16 * S + 8 + 16 * S;
}
constexpr uint64_t kSmallLdsMax = 65536;
// A tile that is not its segment's last holds at least 1023 elements
// (bins_per_tile), so a table within the span limit has at most
// span / 1000 + nseg tiles and nseg + tiles / 1024 scan chunks: its tables
// always fit.
constexpr uint64_t kSmallMaxTiles = ADACOMP_SMALL_TABLE_MAX_SPAN / 1000 + ADACOMP_SMALL_TABLE_MAX_SEGMENTS;
static_assert(small_lds_bytes(kSmallMaxTiles, ADACOMP_SMALL_TABLE_MAX_SEGMENTS + kSmallMaxTiles / 1024 + 1,
                              ADACOMP_SMALL_TABLE_MAX_SEGMENTS) <= kSmallLdsMax,
              "small tables: the finish's tables fit the LDS budget");
// Tables whose compress ends with k_finish_small (and may take the single
// launch): small span, few segments; the LDS tables and the 16-bit ticket
// count are checked as well.
inline bool small_table_fits(const Layout& L) {
    return L.ct.ntiles >= 1 && L.ct.ntiles < 65536 && L.nseg <= ADACOMP_SMALL_TABLE_MAX_SEGMENTS &&
           L.span <= ADACOMP_SMALL_TABLE_MAX_SPAN &&
           small_lds_bytes(L.ct.ntiles, L.ct.nchunks, L.nseg) <= kSmallLdsMax;
}
// The single launch also needs every bin held in registers (tile shapes 0, 1).
inline bool single_launch_fits(const Layout& L) {
    return small_table_fits(L) && L.ct.by_variant[2].empty() &&
           L.ct.by_variant[0].size() + L.ct.by_variant[1].size() == L.ct.ntiles;
}

// LDS bytes of the chunk finish (finalize + encode in one kernel) for C
// scan chunks and S segments: per chunk a double and two words, per segment
// two 64-bit and two 32-bit words, plus one 64-bit total.
ADACOMP_HD constexpr uint64_t chunk_finish_lds_bytes(uint64_t C, uint64_t S) {
    return 8 * C + 8 * C + 16 * S + 8 + 8 * S;
}
// Kept to 32 KB, so that LDS allows the 5 workgroups per CU the kernel's
// registers allow.  A segment of n tiles has ceil(n / 1024) scan chunks, so
// a table within the limits has at most nseg + ntiles / 1024 of them.
constexpr uint64_t kChunkLdsMax = 32768;
static_assert(chunk_finish_lds_bytes(ADACOMP_SMALL_TABLE_MAX_SEGMENTS +
                                         ADACOMP_CHUNK_FINISH_MAX_TILES / kChunkTiles,
                                     ADACOMP_SMALL_TABLE_MAX_SEGMENTS) <= kChunkLdsMax,
              "chunk finish: the chunk and segment tables fit the LDS budget");
inline bool chunk_finish_fits(const Layout& L) {
    return L.ct.ntiles >= 1 && L.ct.ntiles <= ADACOMP_CHUNK_FINISH_MAX_TILES &&
           L.nseg <= ADACOMP_SMALL_TABLE_MAX_SEGMENTS;
}

// How a plan compresses.
enum class Finish { kSeparate, kSmall, kSingle, kChunks };

// The finish a plan made with plan_flags uses (flags already validated).
inline Finish choose_finish(const Layout& L, uint32_t plan_flags) {
    if ((plan_flags & ADACOMP_PLAN_SINGLE_LAUNCH) != 0u && single_launch_fits(L)) return Finish::kSingle;
    if ((plan_flags & ADACOMP_PLAN_SEPARATE_FINISH) != 0u) return Finish::kSeparate;
    if (small_table_fits(L)) return Finish::kSmall;
    if (chunk_finish_fits(L)) return Finish::kChunks;
    return Finish::kSeparate;
}

// Plans whose finish reads the per-tile tables of small_table_fits.
inline bool uses_small_tables(Finish f) { return f == Finish::kSmall || f == Finish::kSingle; }

// Kernel launches of one compress call.
inline uint64_t compress_launches(const Layout& L, Finish f) {
    if (f == Finish::kSingle) return 1;
    uint64_t n = f == Finish::kSmall ? 1 : f == Finish::kChunks ? 2 : 3;   // finish kernels
    for (int v = 0; v < kVariants; ++v) n += L.ct.by_variant[v].empty() ? 0 : 1;
    return n;
}

inline void fill_info(const Layout& L, Finish f, adacomp_plan_info* info) {
    info->nseg = L.nseg;
    info->plan_hash = L.plan_hash;
    info->total_numel = L.total_numel;
    info->span = L.span;
    info->total_bins = L.total_bins;
    info->ntiles = L.ct.ntiles;
    info->header_bytes = 32 + 16 * uint64_t(L.nseg);
    info->message_capacity = L.capacity;
    info->compress_workspace_bytes = L.ws_compress;
    info->decode_workspace_bytes_per_message = L.dws_per_msg;
    info->decode_workspace_bytes_fixed = L.dws_fixed;
    info->compress_launches = compress_launches(L, f);
}

}  // namespace adacomp
