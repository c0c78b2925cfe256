// dispatch_table.hpp -- every width-keyed threshold that the row and column
// entry points choose kernels, tiles and grids by, in one table, each with
// the measurement that chose it (the default launch-shape structs stay next
// to the code in libred.cpp). Host code only (included by libred.cpp).
//
// Unless an entry says otherwise, a figure is from one MI355X on 1 GiB of
// float32 (the 65536 x 4096 uniform[0,1) workload viewed as a contiguous
// (2^28 / cols) x cols matrix), in TB/s of input bytes, with HIP events over
// 20-50 calls; "widths" means `bench.py --widths` (the kernels and per-width
// times of profiles/rows_cols_widths_1gib.md), and "sweep" a launch-shape
// sweep over the named widths run with the `_with` entry points. A change to
// an entry is a change of measured behaviour and should come with a new
// measurement.
#pragma once

#include <stddef.h>

namespace libred {
namespace table {

// ------------------------------------------------------------ rows: choice
// Rows of 1024 floats and more go to a one-wave-per-row kernel; shorter ones
// to the LDS-staged kernel (widths: 1000 floats staged 6.5, one wave per row
// 4.8 TB/s).
constexpr size_t kStagedBelowCols = 1024;
// A staged tile holds at most this many floats (16 loads of 16 bytes per
// lane); contiguous rows whose aligned span does not fit go elsewhere.
constexpr size_t kStagedMaxTileFloats = 4096;
// Strided rows stay staged only under this width (512 floats at a stride of
// 516 ran 6% slower staged than with the packed kernel).
constexpr size_t kStagedStridedBelowCols = 512;
// Strided or unaligned rows up to this width go to the packed kernel (a
// segment of lanes per row) when the staged kernel does not apply.
constexpr size_t kPackedMaxCols = 512;

// ------------------------------------------------------------ rows: narrow kernel
// Rows of up to 32 floats of a contiguous, 16-byte aligned matrix take the
// narrow kernel (each lane folds whole rows): on 1024 waves, against the
// staged kernel with whole-line tiles, TB/s of input plus output, 3 floats
// 5.3-5.4 -> 5.5, 5 floats 5.9 -> 6.1, 7 floats 5.8 -> 6.1, 9-11 floats
// 5.7-5.8 -> 6.0-6.1, 12-15 floats +1-4%, 2, 4, 8 and 16 floats level or
// better (narrow sweep, widths 1-16); the waves by width below add more.
// Widths 17-31 on 1024 waves, medians of three alternating rounds, against
// the staged kernel: odd widths 5.7-5.8 -> 6.0-6.3 TB/s (17: 5.8 -> 6.0-6.1,
// 31: 5.8 -> 6.3), widths 18-30 level to 6% faster. 32 floats, with the
// results held (below): 7.2 / 6.8 TB/s (sum / max) against 6.3-6.4 staged.
constexpr size_t kNarrowDefaultMaxCols = 32;
// Waves by width, from medians of three alternating rounds of sum and max
// (the narrow grid sweep: 256-1536 waves, then 512 against 1024 for every
// width once the result stores were non-temporal). 512 waves, TB/s of input
// plus output against 1024: 1 float 6.1 / 5.9, 3 floats 6.5 / 5.9, 5 floats
// 6.3 / 5.9, 7 floats 6.0-6.2 / 5.9, 9 floats 6.2-6.4 / 5.9, 10 floats
// 6.0-6.1 / 5.9-6.0, 11 floats 6.4 / 6.0, 13 floats 6.1-6.4 / 6.0, 14 floats
// 6.1 / 5.8, 15 floats 6.1-6.3 / 6.0. 1024 waves: 2, 4, 6, 8, 12 and 16
// floats, where 512 ran slower for one operator or both (4 floats 5.5-6.2
// against 6.0-6.2, 8 floats' max 5.6 against 6.2, 16 floats' max 5.2
// against 6.2).
constexpr int kNarrowWaves[kNarrowDefaultMaxCols + 1] = {
    1024, 512,  1024, 512,  1024, 512,  1024, 512,  1024, 512,  512,  512,  1024, 512,  512,  512,
    1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024};
// Widths whose waves hold their results in LDS and store them in bursts,
// on kNarrowHoldWaves waves. TB/s of input plus output, medians of three
// alternating rounds, storing each tile's results (the waves above) against
// holding them on 512 waves, sum / max: 6 floats 5.9-6.0 / 6.2 -> 6.3-6.4 /
// 6.4-6.5 (two machines), 8: 6.1 / 6.1 -> 6.7 / 6.7, 12: 6.0 / 5.9 -> 6.8 /
// 6.9, 16: 6.0 / 6.0 -> 7.0 / 7.0, 21: 6.1 / 6.1 -> 7.1 / 6.5, 25: 6.2 /
// 6.1 -> 6.9 / 6.8, 31: 6.2 / 6.2 -> 6.8 / 6.5; every width from 8 to 32
// gains for both operators (9-15 on a second machine too: +3-10%). Not
// held: 7 floats (+2% on one machine, -5% on another), and below 6 floats,
// whose results are a fifth of the traffic or more (1 float: 6.1 -> 5.5, 3:
// 6.5 -> 6.0, 5: 6.3 -> 5.9 on one machine, level on another). Holding on
// 1024 waves (four per CU where the LDS allows it) ran 2-16% slower than on
// 512, and 768 waves slower still.
constexpr bool kNarrowHold[kNarrowDefaultMaxCols + 1] = {
    false, false, false, false, false, false, true, false, true, true, true, true, true, true, true, true, true,
    true,  true,  true,  true,  true,  true,  true, true,  true, true, true, true, true, true, true, true};
constexpr int kNarrowHoldWaves = 512;

// ------------------------------------------------------------ rows: staged tile
// Tile sizes by the floats a tile's rows span: up to 1024 -> 4 loads per
// lane, up to 2048 -> 8, else 16 (a tile must hold at least one aligned
// span of rows).
constexpr size_t kTileFloats4 = 1024;
constexpr size_t kTileFloats8 = 2048;
// Whole-line tiles (R a multiple of 32 rows) by default under this width:
// 3 floats 4.7 -> 5.4, 5-15 and 17 floats 5.0-5.4 -> 5.7-5.9, 24 floats
// 5.3 -> 5.8 TB/s of input plus output (rows sweep, lines 1 against 2).
constexpr size_t kWholeLinesBelowCols = 32;
// ... and non-power-of-two widths from this one up take 8 loads per lane:
// within 3% of the best of nine shapes at 5-15, 17 and 24 floats; 3 floats
// and the powers of two ran 1-3% faster with 4.
constexpr size_t kWholeLinesWideTileFromCols = 5;
// Rows of whole vectors up to this width read 16-byte vectors from LDS
// (bank conflicts with element reads: 18.7 against 2.0-5.2 cycles per LDS
// instruction at 16 and 64 floats, profiles/rows_staged_lds_counters.md).
constexpr size_t kVectorReadMaxCols = 64;
// Vector-read rows from this width take 4096-float tiles on 1024 waves, and
// 64 floats 2048-float tiles (48: 5.9 -> 6.3, 60: 5.4 -> 6.4, 64: 6.5 -> 6.8).
constexpr size_t kVectorReadBigTileFromCols = 44;
// Element-read rows from 32 to 1023 floats take the largest tile whose
// passes are within this share as full as the fullest tile's (over 54 widths
// of 33-512 floats: 97.3% of the best of four shapes on geometric mean).
// Rows of 513-1023 floats joined the rule together with their lanes per row
// (kWholeWaveAboveCols); see there.
constexpr size_t kElementTileRuleMinCols = 32;
constexpr size_t kElementTileRuleMaxCols = 1023;
constexpr double kPassUseSlack = 0.02;
// Rows of 33-39 floats: 2048-float tiles on 1024 waves when 4096-float tiles
// leave no room to hold the results and their passes are within this share
// as full (sums 5.5 -> 5.5-6.4, maxima 5.5-5.6 -> 5.7-6.0; at 41-43 floats
// the maxima ran 8% slower, so the rule stops below 40).
constexpr size_t kHoldSmallTileBelowCols = 40;
constexpr double kHoldSmallTileSlack = 0.05;
// Waves of the staged kernel: 1024 with 4096-float tiles, else 2048.
constexpr int kStagedBigTileWaves = 1024;
constexpr int kStagedWaves = 2048;
// Lanes per row, element reads: the largest power of two up to cols / 8
// below 32 floats, cols / 16 for whole-vector rows from 128 floats that are
// a multiple of kLanesWholeVecEvenCols floats, else cols / 24 (a sweep of
// lanes per row: 8-16 elements per lane best); rows
// over kWholeWaveAboveCols floats take the whole wave. Rows of 513-1023
// floats took the whole wave and 1024-float tiles (one row per tile); with
// these lanes (16 or 32 per row) and the tile rule above they ran +5.2% on average
// over 12 widths (1 GiB, sums and maxima, two builds alternating: 520: 5.26
// -> 5.80, 640: 6.13 -> 6.96, 900: 6.38 -> 6.92, 1023: 6.43 -> 7.07 TB/s;
// 700, 768, 800 and 960 floats 2-3% slower; they now take their lanes by
// the rows of a tile, below). At 260 and 300 floats 8 lanes
// instead of 16 ran 5% and 24-28% faster, but the divisor that picks them
// (24) cost up to 8.5% at 128, 256, 320 and 512 floats, so whole-vector rows
// take it only when they are not a multiple of 16 floats. Where 16 lanes
// would leave lanes with unequal counts of elements, 24 ran faster (1 GiB,
// two builds alternating, sums / maxima: 140: +10 / +10%, 148: +10 / +13%,
// 276: +19 / +21%, 300: +24 / +28%, 308: +29 / +33%, 372: +5 / +12%;
// 18 of 20 such widths of 132-500 floats within -3% or faster, 132 and 340
// sums -3%); the multiples of 16 were unchanged.
// Rows of kLanesByTileFromCols to kWholeWaveAboveCols floats (element
// reads, 4096-float tiles on 1024 waves) take their lanes by the rows R such
// a tile holds: 16 for R >= 7 (two passes of four rows), 8 for R = 5 and for
// R = 6 below kLanesSixRowsWideFromCols floats (one pass), 32 for R = 6 from
// there (three passes of two rows), 16 for R = 4 below
// kLanesFourRowsWideFromCols floats (one pass) and 32 from there (two
// passes). Sweep on 1 GiB (sums and maxima, medians of three alternating
// rounds of 8, 16 and 32 lanes on 1024 and 2048 waves, 81 widths of 514-1022
// floats of all four residues mod 4): cols / 24 lanes left R = 5 and R = 6
// with 16 (two passes, the second 1/4 or 1/2 full), 10-20% slower than 8
// lanes, and R = 4 with 32 from 768 floats, 3-8% slower than 16 below 900.
constexpr size_t kLanesByTileFromCols = 513;
// Rows of kLanesFourFromCols to 512 floats that are not a multiple of 16
// and whose 4096-float tile holds kLanesFourMinRows to kLanesFourMaxRows
// rows (12 only below kLanesFourMaxRowsBelowCols floats) take 4 lanes per
// row: one pass of up to 16 rows, where cols / 24 lanes (8) took two, the
// second a quarter to a half full. On 1 GiB, two builds alternating (sums /
// maxima): 259: +15 / +22%, 283: +16 / +17%, 314: +15 / +15%, 342: +12 /
// +15%, 350: +14 / +13%, 378: +14 / +20%, 380: +16 / +20%, 33 shapes of
// 259-480 floats +6.6% on geometric mean. With 12 rows from 320 floats
// (324-340) the maxima ran 1-5% slower for sums 0-4% faster, so those keep
// their lanes, as do the multiples of 16.
// In the tile rule for rows of kThinPassFromCols to 512 floats, a tile
// that takes more than one pass with its last at most 1 / kThinPassDivisor
// full yields to the largest smaller tile that takes one pass or fills its
// last better, on 2048 waves. From the sweep of every width (sums and
// maxima against the tile rule's choice, the same lanes): 24 widths changed,
// +9.1% on geometric mean (odd 171-191 floats, 4 lanes, 4096-float tiles
// of 20 rows, passes of 16 and 4 -> 2048-float tiles of 8: +10 to +24%;
// 120 floats: +11%); 112 floats 4-5% slower, every other width faster.
constexpr size_t kThinPassFromCols = 40;
constexpr size_t kThinPassDivisor = 4;
constexpr size_t kLanesFourFromCols = 257;
constexpr size_t kLanesFourMinRows = 10;
constexpr size_t kLanesFourMaxRows = 12;
constexpr size_t kLanesFourMaxRowsBelowCols = 320;
constexpr size_t kLanesSixRowsWideFromCols = 640;
constexpr size_t kLanesFourRowsWideFromCols = 900;
// ... and where such a tile's rows span fewer floats than this (odd widths up
// to 583 floats: four rows), 2048 waves ran 5-7% faster than 1024.
constexpr size_t kStagedSparseTileFloats = 2336;
constexpr size_t kLanesDivNarrow = 8;
constexpr size_t kLanesDivWholeVec = 16;
constexpr size_t kLanesDivOther = 24;
constexpr size_t kLanesNarrowBelowCols = 32;
constexpr size_t kLanesWholeVecFromCols = 128;
constexpr size_t kLanesWholeVecEvenCols = 16;
constexpr size_t kWholeWaveAboveCols = 1023;
// Results held in LDS to the end of the wave under this width (with one or
// two rows per tile, at 960-1020 floats, holding measured 1-10% slower).
constexpr size_t kHoldBelowCols = 960;

// ------------------------------------------------------------ rows: one wave per row
// Rows of at least this many floats take 16 loads per lane on 512 waves
// (sweep over 1024, 4096, 16384 and 65536 floats).
constexpr size_t kRowsLongFromCols = 16384;
constexpr int kRowsLongUnroll = 16;
constexpr int kRowsLongWaves = 512;
// Rows under this width take a tile no longer than the row on 2048 waves.
constexpr size_t kRowsShortBelowCols = 2048;
constexpr int kRowsShortWaves = 2048;
// Rows of 1 to 1.75 tiles of 8 loads per lane (a second tile at most this
// many vectors full) take 4-load tiles on 2048 waves (2052: 4.9 -> 6.4,
// 2560: 5.6 -> 7.1, 3072: 6.2 -> 6.9 TB/s; a 95% full second tile: 3%
// slower).
constexpr size_t kPartialTileMaxVectors = 384;
// Rows read through their aligned covers: 8 loads per lane on up to 32768
// waves below 16384 floats (2049: 5.8 -> 6.8, 2500: 5.5 -> 6.6 TB/s),
// 1024 waves from there (50257 floats: 6% slower on more).
constexpr int kCoverUnroll = 8;
constexpr int kCoverWavesBelowLong = 32768;
constexpr int kCoverWavesLong = 1024;
// Aligned rows under kRowsLongFromCols floats whose last round of loads, in
// the tiles their shape above gives them, is at most this share of a tile
// full are read as covers too, one unconditional tile of 8 loads where the
// row fits, on up to 32768 waves (aligned rows just over 1024 floats paid a
// nearly empty second round per row: 1028: 4.9 -> 6.3, 1060: 5.1 -> 6.4,
// 1200: 5.6 -> 6.5, 1500: 6.3 -> 6.6, 2052: 6.4 -> 6.7, 4100: 6.3 -> 6.8
// TB/s; with a last round 76-100% full (1800, 2048, 6000 floats) the
// covers ran 2-9% slower; 2500 floats, 44%: 1% slower).
constexpr double kCoverLastRoundMax = 0.5;

// ------------------------------------------------------------ rows: split
// Fewer than kSplitRowsBelow rows of at least kSplitMinCols floats are cut
// across blocks, about kSplitTargetWaves waves in all (2 x 2^27: one wave
// per row 27 GB/s, split 7.0 TB/s).
constexpr size_t kSplitRowsBelow = 1024;
constexpr size_t kSplitMinCols = 8192;
constexpr size_t kSplitTargetWaves = 1024;

// ------------------------------------------------------------ rows: strided, staged
// Strided rows of kStagedGapMinCols to kStagedGapMaxCols floats whose gaps
// (ld - cols) hold at most kStagedGapMaxFloats floats go to the LDS-staged
// kernel, which loads the gaps along, like rows whose gaps hold at most a
// quarter of the row; the packed kernel, which reads each row's elements,
// took the rest. Two builds alternating, 1 GiB (2^28 floats of rows of ld),
// TB/s of matrix bytes, packed against staged: 3 at ld 5: 1.7 -> 2.7, 5 at 7:
// 1.5 -> 3.4, 7 at 9: 2.0 -> 3.8, 7 at 16: 1.7 -> 2.5, 12 at 17: 1.7 -> 3.5,
// 17 at 24: 1.2 -> 3.7, 17 at 32: 1.2 -> 3.3, 33 at 48: 1.3 -> 4.0, 40 at
// 64: 2.7 -> 4.1, 60 at 80: 4.2 -> 4.5, 100 at 128: 3.8 -> 5.2, 100 at 150:
// 1.9 -> 4.3 (19 shapes, +6 to +230%). Staged lost where the gaps are long or
// the rows wide (100 at 300: 4.2 -> 2.3, 200 at 300: -13%, 300 at 400:
// -10%, 200 at 256: -3%) and for rows of 1 or 2 floats one float apart
// (-8 to -10%).
constexpr size_t kStagedGapMinCols = 3;
constexpr size_t kStagedGapMaxCols = 128;
constexpr size_t kStagedGapMaxFloats = 64;

// ------------------------------------------------------------ rows: max fold
// The LDS-staged kernel's maxima fold each lane's elements with a hardware
// max of the canonicalized element (v_max3_f32 over two elements, 29
// instructions per 8 elements) instead of a compare and a select through
// an SGPR pair with a wait state between them (41), for rows of fewer than
// this many floats. Two builds alternating over 1 GiB maxima (three rounds,
// spread under 1%): 14 shapes of 33-63 floats +5.7% on average (33: 4.95 ->
// 5.56, 35: 5.47 -> 6.11, 52: 5.63 -> 6.37, 60: 5.66 -> 6.46 TB/s; 33 at an
// unaligned x -4.9%); 64 shapes of 64-1023 floats +2.2% on average but 16
// of them 2-8% slower (64: 6.82 -> 6.50, 65: 6.55 -> 6.11, 100: 6.69 ->
// 6.14, 256: 6.90 -> 6.73), with no launch shape or LDS bank pattern that
// separates them from the gainers (120, 160, 208, 304, 376: +8-13%).
constexpr size_t kStagedMaxFmaxBelowCols = 64;

// ------------------------------------------------------------ rows: XCD grouping
// Rows of kGroupRowsMinCols to kGroupRowsMaxCols - 1 floats that do not all
// start on kRowLineBytes lines are read by grid-stride kernels whose block
// indices are dealt to the XCDs in runs of kGroupRowsChunk consecutive ones
// (grid rounded up to a multiple of 8 runs): a row and the next share the
// line where one ends, and dealt block by block the two waves that read it
// sit on different XCDs and fetch it twice. Sums over 1 GiB, TB/s, launch
// order against runs of 64: contiguous 1000 floats 6.48 -> 6.77, 1020: 6.12
// -> 6.66, 1023: 5.97 -> 6.43, 1025: 6.49 -> 6.97, 1500: 6.54 -> 7.00, 2049:
// 6.86 -> 6.91, 3001: 6.71 -> 7.01; 1000 at ld 1003: 6.37 -> 6.91, 2000 at
// 2001: 6.63 -> 6.99, 1025 at 1028: 5.19 -> 5.34 (+6.4% on average; runs of
// 16 and 256: +6.0% and +6.2%). Elsewhere grouping was neutral or lost: 4097 and 6000
// floats 2% slower, 48 floats 4-7%, whole-line rows (64, 1024, 2048, 4096
// floats) up to 4%; grouping a launch's blocks in 8 contiguous bands (one per
// XCD) lost 6% at 4097 floats, whose bands then lie 64 MiB + 16 KiB apart.
constexpr size_t kGroupRowsMinCols = 768;
constexpr size_t kGroupRowsMaxCols = 4096;
constexpr int kGroupRowsChunk = 64;
constexpr size_t kRowLineBytes = 128;

// ------------------------------------------------------------ columns: folded views
// A width of at least this many columns that is not a multiple of 32 reads
// through views of 32 rows (whole 128-byte lines) when that leaves at least
// kFold32MinViewRows view rows (odd widths 257-4097: 7-17% faster than 16
// rows; 1025: 5.8 -> 6.4, 2049: 5.9 -> 6.9 TB/s).
constexpr size_t kFoldWideFromCols = 256;
constexpr size_t kFold32MinViewRows = 1024;
// Other widths of at least kFoldWideFromCols that are not a multiple of 4:
// 16-row views (1023-65537 columns: 3-24% faster than 4 rows).
constexpr size_t kFold16Rows = 16;
// Widths from 32 to 255: view rows of about kFoldViewFloats floats (512
// groups of four columns), at most kFoldMaxRows rows (33: 5.6 -> 6.7, 65:
// 5.5 -> 6.8 TB/s), unless a multiple of 4 already uses this share of the
// lanes.
constexpr size_t kFoldMidFromCols = 32;
constexpr size_t kFoldViewFloats = 2048;
constexpr size_t kFoldMaxRows = 64;
constexpr double kFoldMidLaneUse = 0.95;
// Under 32 columns: the smallest line-spanning view keeping this share of
// the lanes busy (23: 5.7 -> 6.3, 28: 6.1 -> 6.5, 31: 6.1 -> 6.8 TB/s),
// unless the best view up to 16 rows already keeps kFoldNarrowEnough.
constexpr double kFoldNarrowLaneUse = 0.84;
constexpr double kFoldNarrowEnough = 0.99;
// A multiple of 4 is folded only when that uses this much more of the lanes
// (260 columns: 4.0 -> 6.4 TB/s folded 16 rows).
constexpr double kFoldGain = 0.05;

// ------------------------------------------------------------ columns: row order
// Rows read at a pitch (the matrix's leading dimension, or the view's) that
// is a multiple of one of these many floats start each block's sweep at a
// different row group (rotated order) instead of sweeping one band of the
// matrix: with the band, every one of these pitches read at 5.0-5.7 TB/s
// against 6.1-7.1 for the neighbouring widths (1012-1036, 2032-2052,
// 3052-3068, 4080-4084, 5096-5104, 6120-6124, 8160-8164 columns and
// 508-516, 765-766, 1530-1534), and the DRAM credit stalls per read request
// rose from 0.02-0.03 to 0.19-0.49 (TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum at
// 1020, 1028 and 2040 columns). Rotated, sums of 1020, 2040, 3060, 4080,
// 5100, 6120, 7140 and 8160 columns read at 5.9-6.3 TB/s (+0.5-0.9), 510,
// 765 and 1530 columns (32640- and 97920-byte view rows) at 6.0-6.2 (+0.5),
// 1028, 2056, 3084 and 4112 at 5.4-5.6 (+0.1-0.4); at the other widths of
// that scan the rotated order ran up to 3% slower, so it stays off there.
// That holds for the views (32-row views of 765, 2040, 2056, 3060, 3084,
// 4080 and 5100 columns: rotated 4-15% faster than runs of rows, with the
// blocks grouped per XCD). A matrix read unfolded at such a pitch takes one
// run of rows per phase instead: with the XCD grouping, runs against
// rotated, sums TB/s, 1024 columns at ld 1028: 6.23 -> 6.87, 2000 at 2056:
// 6.11 -> 6.65, 1016 at 1020: 6.14 -> 6.85, 508 at 510: 6.04 -> 6.54, 500 at
// 514: 5.97 -> 6.42, 512 at 514: 4.87 -> 5.13, 4096 at 4112: 6.21 -> 6.41,
// contiguous 8160 (unfolded): 6.31 -> 6.57; 255 and 256 at ld 257 within
// 2% either way.
constexpr size_t kRotateRowsPitchFactorA = 255;
constexpr size_t kRotateRowsPitchFactorB = 257;
// A narrow matrix (or view) whose wave loads each cover several rows
// (ngroups < 64) takes one run of consecutive rows per phase when such a
// load's rows do not span whole lines of this many bytes: in the band order
// the line at each boundary between two loads' rows is read by two waves of
// different phases (on different XCDs) and fetched twice (1.07-1.14 times
// the input at 3, 12, 17 and 24 columns); in a run the next load is the same
// wave's. Sums, TB/s of input, band against runs: 3 columns 6.1 -> 6.9, 5:
// 6.5 -> 7.0, 6: 6.1 -> 6.9, 9: 6.1 -> 6.9, 11: 6.1 -> 6.9, 12: 6.0 -> 6.8,
// 13: 6.3 -> 6.8, 17: 6.0 -> 6.6, 18: 6.1 -> 7.0, 20: 6.5 -> 6.9, 24: 6.5 ->
// 6.9, 25: 6.1 -> 6.5 (maxima alike); where the loads span whole lines (1,
// 2, 4, 8, 16 and 32 columns, and the line-spanning views of 7, 15, 21-23
// and 27-31 columns) runs read 1-4% slower, so the band stays there.
constexpr size_t kLineBytes = 128;

// ------------------------------------------------------------ columns: XCD grouping
// A launch of at least this many row phases deals each XCD the column
// blocks of a run of consecutive phases (the phases rounded down to a
// multiple of 8), unless the row pitch as read (ld or the view's) is a
// power of two bytes. Where rows, or a block's share of a row, do not end on
// a 128-byte line, two blocks read the line between them, and it is fetched
// twice when they run on different XCDs: sums over 1 GiB matrices read
// 1.06-1.11 times their input dealt block by block, 1.04-1.05 grouped; 4096
// columns at ld 4097: 5.3 -> 6.3 TB/s, 3000 at 3001: 5.4 -> 6.6, 1020 at
// 1021: 4.7 -> 6.4, 8192 at 8193: 5.1 -> 6.3, 4096 at 4100: 6.2 -> 6.6, 1024
// at 1028: 5.2 -> 6.2, 256 at 257: 5.3 -> 5.5; contiguous 100 and 260
// columns +12% and +5%, the other contiguous widths from 1 to 2^20 within 1%.
// At power-of-two pitches (contiguous 1, 4, 16, 32, 64, 256, 512, 1024, 4096
// and 16384 columns, 1000 columns at ld 1024) grouping ran 5-7% slower.
constexpr size_t kXcdGroupMinPhases = 8;
// Folded views (m-row views of 256 or more columns) of at most this many
// 256-column blocks whose default launch (512 waves) leaves too few row
// phases to be grouped per XCD take 4 rows in flight on 1024 waves
// (kFoldPhasesCols), which gives them 5 or more phases, grouped from 8. On
// 1 GiB (sums and maxima, medians of three alternating rounds), 22 such
// widths of 276-1756 columns (35-220 blocks of their 32-row views): +3.6%
// on geometric mean (340: 5.6 / 5.5 -> 6.2 / 6.4, 1052: 5.4 / 5.5 -> 6.0 /
// 6.2, 1700: 5.4 / 5.4 -> 6.4 / 6.6 TB/s; worst 652 columns, -4 / -5%).
// Over 20 widths of 1800-2556 columns (225-320 blocks) it came to -0.4%,
// with 1900 and 2350 columns 9-11% slower, so wider views keep the default.
constexpr size_t kFoldFewPhasesMaxBlocks = 224;
// Unfolded rows of more than this many columns, up to kWideColBlocks blocks
// of 256, at a pitch that is not a power of two bytes, take 4 rows in flight
// with 2 KiB of a row per wave on 1024 waves (kUnfoldedWideCols). Multiples
// of 32 there had 7-11 row phases under the default, too few to group per
// XCD, and other widths took the short-wide shape. Sweep of 54 shapes on
// 1 GiB, sums / maxima against those: 12000: +8.6 / +7.2%, 20000: +8.0 /
// +5.8%, 100000: +5.3 / +6.4%, 8200: +4.8 / +0.6%, 9000: +4.7 / +1.9%, 10000:
// +2.6 / +0.3%, 200000: +2.6 / +2.7%. Where the shape it replaces has its
// blocks grouped per XCD and this one would not, the old shape stays (50000
// columns: 21 phases grouped against 11 not, 6% slower).
constexpr size_t kUnfoldedWideAboveCols = 8192;
// ... and only when rounding the phases down to a multiple of 8 keeps this
// share of them: 300 contiguous columns (38 blocks per view row, 14 phases,
// cut to 8) ran 16-25% slower grouped. Rounding up instead lost more where
// the default grids sit just under 1024 single-wave blocks (4 per CU): 9
// blocks per row and 120 phases instead of 112 took 4096 columns at ld 4097
// from 6.3 to 4.7 TB/s, 1020 at 1021 (344 phases instead of 336) from 6.4
// to 4.6, as the grid passed 1024 and some CUs held a fifth wave.
constexpr double kXcdGroupKeepPhases = 0.75;
// Launches with fewer phases stay in launch order. Grouping them as well
// (contiguous ranges of column blocks per XCD, any grid) was measured on 16-row
// views of odd widths, one or two phases each: +2 to +4% at 20001, 24577,
// 50257 and 100003 columns, -4 to -8% at 8193, 12289, 16385, 65537 and
// 131073, whose view pitches lie 64 bytes past a multiple of 256 KiB.

// ------------------------------------------------------------ columns: shapes
// Short-wide matrices (more than this many blocks of 256 columns), and rows
// of at least kFoldWideFromCols columns that are not whole lines (unfolded),
// take the wide shape (256 x 1M: 5.9 -> 7.1 TB/s; 1020, 1500, 3000, 6000
// columns 8-12% faster).
constexpr size_t kWideColBlocks = 1024;
// The short-wide shape rounds its row phases down so that the grid holds at
// most this many single-wave blocks (4 per CU); rounded up, 16385, 30001
// and 50257 columns took 1028, 1407 and 1572. Where that leaves at most
// kShortWidePrefetchMaxWaves blocks (about 2 per CU), the prefetch goes on.
// On 1 GiB, two builds alternating (sums / maxima, medians of three
// rounds): 20001: +4 / +4%, 24577: +8 / -3%, 30001: +9 / +8%, 50257: +10 /
// +3%, 300000: +8 / +4%, 524292 (513 blocks, prefetch): +14 / +8%, 40003
// (626 blocks, prefetch): 0 / -1%; without the prefetch 524292 and 40003
// ran 6-29% slower.
constexpr int kShortWideMaxWaves = 1024;
constexpr int kShortWidePrefetchMaxWaves = 640;
// The unfolded-wide shape (kUnfoldedWideAboveCols) with at least this many
// blocks per phase rounds its phases down too, where the rounded grid keeps
// at least kUnfoldedRoundMinWaves blocks (or leaves at most
// kShortWidePrefetchMaxWaves, with the prefetch). Sums / maxima against
// rounding up: 100000 columns (980 blocks): +9 / +9%, 150000 (879): +7 /
// +6%, 250000 (978): +6 / +7%, 262148 (513, prefetch): +15 / +15%. At 704
// and 782 blocks (180000, 200000 columns) it ran 2-12% slower without the
// prefetch and 0-3% faster or 7-9% slower with it, so those keep their
// grids; with fewer blocks per phase (24000 columns, 47 blocks in 21
// phases) the maxima ran 9% slower.
// Column maxima fold with a hardware max of the canonicalized element
// instead of a compare and a select in folded views of fewer than this many
// real columns and in short-wide matrices. Two builds alternating, 1 GiB,
// maxima: 7 columns +5%, 17: +8%, 33: +3%, 65: +4%, 100: +4%, 50257: +6%;
// at 260, 1000, 1025, 4096 and 100000 columns it ran 1-1.5% slower, so
// those keep the compare and select.
constexpr size_t kColsFmaxBelowCols = 256;
constexpr size_t kUnfoldedRoundMinBlocks = 128;
constexpr size_t kUnfoldedRoundMinWaves = 864;

}  // namespace table
}  // namespace libred
