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
// The kernels live in common.hpp (shared helpers), tile_pass.hpp, encode.hpp,
// small_table.hpp and decode.hpp; this header includes them all.
//
// Compress, per call, up to four stream-ordered launches (small tables: the
// tile pass and one finish kernel that does the work of the last three, see
// small_table.hpp; tables of up to 256 segments and 2^20 tiles: the tile
// pass, the chunk scan and k_finish_chunks, finalize and encode in one):
//   tile pass   (dense, one workgroup per tile of whole bins; bins longer than
//               4093 elements one per workgroup, streamed twice): reads residue
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
// in order in LDS (long bins: directly in out) and writes each tile once, or,
// fused with an optimizer, takes one SGD or Adam step on the weights instead.
#pragma once

#include "common.hpp"
#include "tile_pass.hpp"
#include "encode.hpp"
#include "small_table.hpp"
#include "decode.hpp"
