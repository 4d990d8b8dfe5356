// Host-side check of the work decomposition the HIP kernels rely on, using
// the library's own layout code (layout.hpp is plain C++).  For every segment
// table read from the input file it verifies, tile by tile and for both the
// compress tiles and the decode tiles, that every access the kernels derive
// from the tile geometry stays inside its buffer and its LDS allocation, that
// the tiles partition each segment exactly, and that the multiply-high bin
// division is exact for every in-tile offset.
//
// Input: blocks of "nseg expected_status" followed by nseg lines
// "offset numel bin_len".  Output: one line per table, "OK ..." or
// "FAIL <reason>"; exit status 1 if any table fails.
#include <cstdio>
#include <cstdint>
#include <string>
#include <vector>

#include "../../adaptive_residual_gradient_amd/csrc/layout.hpp"

using namespace adacomp;

// capacity and threads x float4-per-thread of shape v of a tiling
struct Shapes {
    uint32_t cap[3];
    uint32_t lanes_vecs[3];
    int n;
};

static std::string check_tiling(const Layout& L, const Tiling& T, bool decode, const Shapes& sh) {
    uint64_t seen = 0;
    for (uint32_t s = 0; s < L.nseg; ++s) {
        const SegDev& d = L.segs[s];
        const TileSpec& ts = decode ? d.dt : d.ct;
        if (int(ts.variant) >= sh.n) return "FAIL variant";
        if (!decode && ts.variant == 2 && ts.bpt != 1) return "FAIL long bins share a tile";
        if (ts.bpt == 0 || ts.bpt > T.max_bpt[ts.variant]) return "FAIL bpt";
        for (uint32_t v = 0; v < ts.variant; ++v)
            if (d.lt + 3 <= sh.cap[v]) return "FAIL shape not the smallest";
        uint64_t next = d.off;
        uint32_t next_bin = 0;
        for (uint32_t t = ts.tile_begin; t < ts.tile_begin + ts.ntiles; ++t) {
            if (T.tile_seg[t] != s) return "FAIL tile_seg";
            const TileGeom g = tile_geom(d, ts, t);
            if (g.t0 != next || g.first_bin != next_bin) return "FAIL partition";
            if (g.nb == 0 || g.nb > ts.bpt || g.tlen == 0) return "FAIL empty tile";
            if (g.t0 + g.tlen > d.off + d.numel) return "FAIL tile past segment end";
            if (g.v0 + 4 * uint64_t(g.nvec) > L.span) return "FAIL float4 past padded span";
            if (g.nvec > sh.lanes_vecs[ts.variant]) return "FAIL vectors exceed threads";
            if (uint64_t(g.nvec) * 4 > sh.cap[ts.variant]) return "FAIL vectors exceed cap";
            if (g.nvec > T.max_span_vecs[ts.variant]) return "FAIL LDS tile too small";
            if (g.lead + g.tlen >= 65536u) return "FAIL offsets exceed 16 bits";
            if ((g.t0 & 3) != g.lead || g.v0 % 4 != 0) return "FAIL lead";
            if (g.first_bin + g.nb < d.nbins && g.tlen != uint64_t(g.nb) * d.lt) return "FAIL partial bin";
            for (uint32_t x = 0; x < g.tlen + g.lead; ++x)
                if (div_bin(x, d.lt, d.magic) != x / d.lt) return "FAIL div_bin";
            const uint64_t cw_end = d.count_off + uint64_t(g.first_bin + g.nb) * d.wb;
            if (cw_end > d.count_off + uint64_t(d.nbins) * d.wb) return "FAIL count words";
            next = g.t0 + g.tlen;
            next_bin = g.first_bin + g.nb;
            ++seen;
        }
        if (next != d.off + d.numel || next_bin != d.nbins) return "FAIL coverage";
        for (uint32_t c = ts.chunk_begin; c < ts.chunk_begin + ts.nchunks; ++c) {
            if (T.chunk_seg[c] != s) return "FAIL chunk_seg";
            const uint32_t a = T.chunk_tile_begin[c], b = T.chunk_tile_begin[c + 1];
            if (b <= a || b - a > T.chunk_tiles || T.chunk_tiles > kChunkTiles) return "FAIL chunk size";
            if (a < ts.tile_begin || b > ts.tile_begin + ts.ntiles) return "FAIL chunk crosses segment";
            if ((a - ts.tile_begin) / T.chunk_tiles != c - ts.chunk_begin) return "FAIL chunk index";
        }
    }
    if (seen != T.ntiles || T.chunk_tile_begin.back() != T.ntiles) return "FAIL tile count";
    uint64_t in_variants = 0;
    for (int v = 0; v < 3; ++v) in_variants += T.by_variant[v].size();
    if (in_variants != T.ntiles) return "FAIL variants";
    return "";
}

static std::string check(const std::vector<adacomp_segment>& segs, int expect_status) {
    Layout L;
    const int st = build_layout(segs.data(), static_cast<uint32_t>(segs.size()), L);
    if (st != expect_status) return "FAIL status " + std::to_string(st);
    if (st != ADACOMP_OK) return "OK rejected";
    if (L.span % 4 != 0) return "FAIL span not padded";
    Shapes cs{}, ds{};
    cs.n = kVariants;
    for (int v = 0; v < kVariants; ++v) {
        cs.cap[v] = var_cap(v);
        // shape 2 streams its one bin in chunks
        cs.lanes_vecs[v] = v == 2 ? kLongCap / 4 : kVarThreads[v] * kVarVecs[v];
    }
    ds.n = kDecVariants;
    ds.cap[0] = kDecCap;
    ds.lanes_vecs[0] = kDecCap / 4;   // decode walks float4 with a strided loop
    ds.cap[1] = kMaxCap;
    ds.lanes_vecs[1] = kMaxCap / 4;
    std::string r = check_tiling(L, L.ct, false, cs);
    if (!r.empty()) return r + " (compress tiles)";
    r = check_tiling(L, L.dt, true, ds);
    if (!r.empty()) return r + " (decode tiles)";
    for (const SegDev& d : L.segs)
        if (round_up(d.count_off + uint64_t(d.nbins) * d.wb, 16) > L.entries_begin) return "FAIL count region";
    uint64_t at = L.entries_begin;
    for (const SegDev& d : L.segs) at = round_up(at + d.numel * d.wb, 16);
    if (at != L.capacity) return "FAIL capacity";
    if (L.ws_tile_cnt - L.ws_stage < 4 * L.span) return "FAIL stage size";   // one 32-bit key per element
    // LDS per workgroup stays within 64 KiB.
    for (int v = 0; v < kVariants; ++v)
        if (!L.ct.by_variant[v].empty() && (2 * L.ct.max_bpt[v] + 1) * 4 > 65536) return "FAIL tile LDS";
    for (int v = 0; v < kDecVariants; ++v) {
        if (L.dt.by_variant[v].empty()) continue;
        const uint32_t ps = L.dt.max_bpt[v] + 1;
        const uint32_t kg = decode_group(ADACOMP_MAX_MESSAGES, ps);
        if (kg > 64 || kg * ps > kPrefWords) return "FAIL decode group";
        const uint32_t acc = v == 0 ? L.dt.max_span_vecs[0] * 4 : 0;
        if (decode_lds_bytes(acc, ADACOMP_MAX_MESSAGES, kg, ps, kDecThreads[v] / 64) > 65536)
            return "FAIL decode LDS";
        if (v == 0) {
            const uint32_t tg = decode_tiles_group(ADACOMP_MAX_MESSAGES, ps);
            // with the largest bin-start table a plain decode reserves
            if (decode_tiles_lds_bytes(acc, ADACOMP_MAX_MESSAGES, tg, ps, true, kTblBytes / 4) > 65536)
                return "FAIL decode tiles LDS";
            // the plain sum of up to kMaskMsgs messages, where they fit one group
            if (decode_tiles_group(kMaskMsgs, ps) == kMaskMsgs &&
                decode_sum_lds_bytes(acc, kMaskMsgs, ps) > 65536)
                return "FAIL decode sum LDS";
        }
    }
    // The decode launch order (runs of kXcdGroup positions per XCD) is a
    // bijection of the launch positions, for this table's LDS decode tiles
    // and for every n up to 300.
    {
        std::vector<uint64_t> ns = {L.dt.by_variant[0].size()};
        for (uint64_t n = 1; n <= 300; ++n) ns.push_back(n);
        for (uint64_t n : ns) {
            std::vector<char> seen(n, 0);
            for (uint64_t b = 0; b < n; ++b) {
                const uint32_t p = xcd_grouped(uint32_t(b), uint32_t(n));
                if (p >= n || seen[p]) return "FAIL xcd order n=" + std::to_string(n);
                seen[p] = 1;
            }
        }
    }
    return "OK tiles=" + std::to_string(L.ct.ntiles) + " dtiles=" + std::to_string(L.dt.ntiles);
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
