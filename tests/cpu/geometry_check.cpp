// Host-side check of the work decomposition the HIP kernels rely on, using
// the library's own layout code (layout.hpp is plain C++).  For every segment
// table read from the input file it verifies, tile by tile, that every access
// the kernels derive from the tile geometry stays inside its buffer and its
// LDS allocation, that the tiles partition each segment exactly, and that the
// multiply-high bin division is exact for every in-tile offset.
//
// Input: blocks of "nseg" followed by nseg lines "offset numel bin_len".
// Output: one line per table, "OK ..." or "FAIL <reason>"; exit status 1 if
// any table fails.
#include <cstdio>
#include <cstdint>
#include <string>
#include <vector>

#include "../../adaptive_residual_gradient_amd/csrc/layout.hpp"

using namespace adacomp;

static std::string check(const std::vector<adacomp_segment>& segs, int expect_status) {
    Layout L;
    const int st = build_layout(segs.data(), static_cast<uint32_t>(segs.size()), L);
    if (st != expect_status) return "FAIL status " + std::to_string(st);
    if (st != ADACOMP_OK) return "OK rejected";
    uint64_t tiles_seen = 0;
    for (uint32_t s = 0; s < L.nseg; ++s) {
        const SegDev& d = L.segs[s];
        if (d.bpt == 0 || d.bpt > L.max_bpt[d.variant]) return "FAIL bpt";
        uint64_t next = d.off;       // tiles must cover the segment in order
        uint32_t next_bin = 0;
        for (uint32_t t = d.tile_begin; t < d.tile_begin + d.ntiles; ++t) {
            if (L.tile_seg[t] != s) return "FAIL tile_seg";
            const TileGeom g = tile_geom(d, t);
            if (g.t0 != next || g.first_bin != next_bin) return "FAIL partition";
            if (g.nb == 0 || g.nb > d.bpt || g.tlen == 0) return "FAIL empty tile";
            if (g.t0 + g.tlen > d.off + d.numel) return "FAIL tile past segment end";
            if (g.t0 + g.tlen > L.span) return "FAIL tile past span";
            // whole-float4 loads (lanes past the tile reload its last float4)
            if (g.v0 + 4 * uint64_t(g.nvec) > L.span) return "FAIL float4 past padded span";
            if (L.span % 4 != 0) return "FAIL span not padded";
            if (g.nvec > kVarThreads[d.variant] * kVarVecs[d.variant]) return "FAIL vectors exceed threads";
            if (uint64_t(g.nvec) * 4 > var_cap(int(d.variant))) return "FAIL vectors exceed cap";
            // the first shape that holds the bin is used
            for (uint32_t v = 0; v < d.variant; ++v)
                if (d.lt + 3 <= var_cap(int(v))) return "FAIL shape not the smallest";
            if (g.nvec > L.max_span_vecs[d.variant]) return "FAIL decode LDS too small";
            if (g.lead + g.tlen >= 65536u) return "FAIL offsets exceed 16 bits";
            if ((g.t0 & 3) != g.lead || g.v0 % 4 != 0) return "FAIL lead";
            // every bin except the last of the segment is whole
            if (g.first_bin + g.nb < d.nbins && g.tlen != uint64_t(g.nb) * d.lt) return "FAIL partial bin";
            // exact division for every in-tile offset
            for (uint32_t x = 0; x < g.tlen; ++x)
                if (div_bin(x, d.lt, d.magic) != x / d.lt) return "FAIL div_bin";
            // count words of the tile stay in the segment's count region
            const uint64_t cw_end = d.count_off + uint64_t(g.first_bin + g.nb) * d.wb;
            if (cw_end > d.count_off + uint64_t(d.nbins) * d.wb) return "FAIL count words";
            next = g.t0 + g.tlen;
            next_bin = g.first_bin + g.nb;
            ++tiles_seen;
        }
        if (next != d.off + d.numel || next_bin != d.nbins) return "FAIL coverage";
        if (round_up(d.count_off + uint64_t(d.nbins) * d.wb, 16) > L.entries_begin) return "FAIL count region";
        // chunks of this segment
        for (uint32_t c = d.chunk_begin; c < d.chunk_begin + d.nchunks; ++c) {
            if (L.chunk_seg[c] != s) return "FAIL chunk_seg";
            const uint32_t a = L.chunk_tile_begin[c], b = L.chunk_tile_begin[c + 1];
            if (b <= a || b - a > kChunkTiles) return "FAIL chunk size";
            if (a < d.tile_begin || b > d.tile_begin + d.ntiles) return "FAIL chunk crosses segment";
            if ((a - d.tile_begin) / kChunkTiles != c - d.chunk_begin) return "FAIL chunk index";
        }
    }
    if (tiles_seen != L.ntiles || L.chunk_tile_begin.back() != L.ntiles) return "FAIL tile count";
    // worst-case message fits its capacity
    uint64_t at = L.entries_begin;
    for (const SegDev& d : L.segs) at = round_up(at + d.numel * d.wb, 16);
    if (at != L.capacity) return "FAIL capacity";
    // staging: survivor slots t0 + rank < t0 + tlen <= span, inside the stage buffer
    if (L.ws_tile_cnt - L.ws_stage < 8 * L.span) return "FAIL stage size";
    // LDS per workgroup (bytes) stays within 64 KiB: decode keeps narrow and
    // medium tiles in LDS; the tile pass holds 2*bpt+1 words.
    uint64_t tiles_in_variants = 0;
    for (int v = 0; v < kVariants; ++v) {
        tiles_in_variants += L.tiles_by_variant[v].size();
        if (L.tiles_by_variant[v].empty()) continue;
        const uint32_t ps = L.max_bpt[v] + 1;
        const uint32_t kg = std::max<uint32_t>(1, std::min<uint32_t>(ADACOMP_MAX_MESSAGES, kPrefWords / ps));
        if (v < 2 && (L.max_span_vecs[v] * 4 + kg * ps) * 4 > 65536) return "FAIL decode LDS";
        if (v == 2 && kg * ps * 4 > 65536) return "FAIL decode LDS";
        if ((2 * L.max_bpt[v] + 1) * 4 > 65536) return "FAIL tile LDS";
    }
    if (tiles_in_variants != L.ntiles) return "FAIL variants";
    return "OK tiles=" + std::to_string(L.ntiles) + " chunks=" + std::to_string(L.nchunks);
}

int main(int argc, char** argv) {
    if (argc < 2) return 2;
    FILE* f = std::fopen(argv[1], "r");
    if (!f) return 2;
    int bad = 0;
    unsigned n;
    int expect;
    while (std::fscanf(f, "%u %d", &n, &expect) == 2) {
        std::vector<adacomp_segment> segs(n);
        for (unsigned i = 0; i < n; ++i) {
            unsigned long long o, m;
            unsigned lt;
            if (std::fscanf(f, "%llu %llu %u", &o, &m, &lt) != 3) return 2;
            segs[i] = adacomp_segment{o, m, lt, 0};
        }
        const std::string r = check(segs, expect);
        std::printf("%s\n", r.c_str());
        if (r.rfind("FAIL", 0) == 0) bad = 1;
    }
    std::fclose(f);
    return bad;
}
