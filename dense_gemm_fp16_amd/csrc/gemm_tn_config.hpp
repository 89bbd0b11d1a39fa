// Tile configurations: the k-depth BK, the LDS ring depth and the MFMA
// block edge of each tile shape.  Shared by the host planner and the kernel
// instantiations; the macros exist so that tuning builds can try other
// values.
#pragma once

#ifndef GTN_T256_BK
#define GTN_T256_BK 64
#endif
#ifndef GTN_T256_STAGES
#define GTN_T256_STAGES 2
#endif
#ifndef GTN_T256_WM
#define GTN_T256_WM 2
#endif
#ifndef GTN_T256_WN
#define GTN_T256_WN 4
#endif
#ifndef GTN_T256_MINW
#define GTN_T256_MINW 2
#endif
#ifndef GTN_T256_SCHED
#define GTN_T256_SCHED 2
#endif
#ifndef GTN_T128_BK
#define GTN_T128_BK 64
#endif
#ifndef GTN_T128_STAGES
#define GTN_T128_STAGES 2
#endif
// The 64 tile takes 128-deep k-tiles (rows of 256 bytes) for whole-K
// problems, 64-deep ones for split-K slices: measured (kernel trace, one
// box), 1024^3 with C ran 6.7-7.5 us against 8.0-8.1 us with 64-deep
// tiles, 1000x1030x1000 and 256^3 the same; the 128x4096x8192 slices
// gained nothing from 128 (16.6 against 16.4 us).
#ifndef GTN_T64_BK
#define GTN_T64_BK 128
#endif
#ifndef GTN_T64_SPLIT_BK
#define GTN_T64_SPLIT_BK 64
#endif
// The 64 tile runs short K loops of small problems with a two-stage ring,
// and split-K slices (long loops, two workgroups per CU) with four stages:
// measured, two stages took 1024^3 with C from 8.3 to 7.7 us and
// 1000x1030x1000 from 10.2 to 9.4 us, while the 128x4096x8192 slices went
// from 20.8 to 23.6 us.
#ifndef GTN_T64_STAGES
#define GTN_T64_STAGES 2
#endif
#ifndef GTN_T64_SPLIT_STAGES
#define GTN_T64_SPLIT_STAGES 4
#endif
#ifndef GTN_T256_MFMA
#define GTN_T256_MFMA 16
#endif
#ifndef GTN_T128_MFMA
#define GTN_T128_MFMA 16
#endif
#ifndef GTN_T64_MFMA
#define GTN_T64_MFMA 16
#endif
// Four-wave schedule of the 256 tile (TN operands, direct loads): the MFMA
// of k-step 1 after which the tile's barrier sits, and the slots of the 16
// tile loads in k-step 0 (after MFMA LOAD_FIRST + LOAD_EVERY * x).
// Measured at 4096^3 (HIP events, one box, the ping-pong kernel interleaved
// as the yardstick): loads every 4 MFMAs beat every 3, 2 or 1 (a burst of
// 16 at the start of the k-step was 11 % slower); the barrier after MFMA
// 32, 40 or 47 made no difference beyond noise.
#ifndef GTN_W4_BARRIER_AT
#define GTN_W4_BARRIER_AT 47
#endif
#ifndef GTN_W4_LOAD_FIRST
#define GTN_W4_LOAD_FIRST 3
#endif
#ifndef GTN_W4_LOAD_EVERY
#define GTN_W4_LOAD_EVERY 4
#endif
// Most rows a wave stages through LDS per epilogue pass: with several
// passes the stores of one pass leave while the next is staged.
#ifndef GTN_EPI_MAX_RPP
#define GTN_EPI_MAX_RPP 32
#endif
// Cache-policy bits of the staged 16-byte output stores of the one-k-tile
// and attention kernels (gfx950: 1 = sc0, 2 = nt, 16 = sc1).
#ifndef GTN_STORE_CPOL
#define GTN_STORE_CPOL 2
#endif
// Cache-policy bits of the tile kernels' staged output (and split-K
// partial) stores: sc1.  Measured against streaming (nt) stores with one
// staging pass (HIP events, both builds interleaved in one process, same
// box; bit-identical results), 32-row passes with sc1 stores took 4096^3
// from 97.2-98.0 to 96.6-97.2 us, 4096 x 4096 x 1024 29.95 -> 29.13,
// 128 x 4096 x 8192 (split) 20.5 -> 19.9, 1024^3 (fp32, C) 6.52 -> 6.29,
// 1000 x 1030 x 1000 9.29 -> 8.89, 2048^3 24.0 -> 23.5; default-policy
// stores were slower than either.  The one-k-tile kernel keeps nt stores
// (sc1: 48.2 against 44.7-46.0 us on the score product).
#ifndef GTN_TILE_STORE_CPOL
#define GTN_TILE_STORE_CPOL 16
#endif
// Operand storages each tile has kernels for (bit L = layout L: bit 0 set
// = A stored along M, bit 1 = B stored along N).  Direct loader: the
// transposing LDS reads exist for 16x16 MFMA tiles, every layout.
// Element loader: every layout, except on the 256-wide tile (spills).
#define GTN_T256_DIRECT_LAYS (GTN_T256_MFMA == 16 ? 0xF : 0x1)
#define GTN_T128_DIRECT_LAYS (GTN_T128_MFMA == 16 ? 0xF : 0x1)
#define GTN_T64_DIRECT_LAYS (GTN_T64_MFMA == 16 ? 0xF : 0x1)
#define GTN_T256_ELEM_LAYS false
#define GTN_T128_ELEM_LAYS true
#define GTN_T64_ELEM_LAYS true
