// l9_catalogue.h -- a catalogue of legal configurations of level 9's tile
// template (l9_tile.h), compiled for tuning sweeps and reached through
// hip_sgemm_tile_split's tile ids after the seven named tiles.
//
// [GEMM2] (autotuning section) tunes its kernel's template parameters --
// block tile BM x BN, stage depth BK, per-thread tile TM x TN -- over every
// combination that the kernel's constraints allow, and finds that the best
// set differs from GPU to GPU, so it is searched, not derived.  The
// parameters of this template are the block tile BM x BN, the stage depth
// BK, the wavefront grid WAVES_M x WAVES_N (each wavefront's tile is
// (BM / WAVES_M) x (BN / WAVES_N), the counterpart of TM x TN one level up),
// the matrix instruction (16 x 16 x 4 or 32 x 32 x 2 blocks), K slices per
// stage, and prefetch depth.  The template's static_asserts are the
// legality constraints: wavefront tiles whole in blocks, at most four blocks
// per wavefront per dimension, a stage whole in MFMA steps and split evenly
// over the K slices, every operand panel staged evenly by the block's
// threads, rows of whole 64-word multiples; the configurations below are
// legal ones that span those parameters.
//
// Each entry: X(index, name, BM, BN, BK, WAVES_M, WAVES_N, UNROLL, GROUP_M,
// PRIO, KSLICE, DEPTH, MS).  Names give BM x BN x BK, the wavefront grid,
// the matrix block size and the K slices.
#pragma once

#define SGEMM_CATALOGUE_FIRST(X)                                                  \
  X(0, "cat_64x64x32_1x1w_m16", 64, 64, 32, 1, 1, 16, 8, false, 1, 1, 16)        \
  X(1, "cat_64x64x16_2x2w_m16", 64, 64, 16, 2, 2, 8, 8, false, 1, 1, 16)         \
  X(2, "cat_64x128x16_1x2w_m16", 64, 128, 16, 1, 2, 8, 8, false, 1, 1, 16)       \
  X(3, "cat_128x64x16_2x1w_m16", 128, 64, 16, 2, 1, 8, 8, false, 1, 1, 16)       \
  X(4, "cat_128x64x32_2x2w_m16_2slices", 128, 64, 32, 2, 2, 16, 8, false, 2, 1, 16)

#define SGEMM_CATALOGUE_SECOND(X)                                                 \
  X(5, "cat_128x128x16_2x2w_m16", 128, 128, 16, 2, 2, 8, 8, false, 1, 1, 16)     \
  X(6, "cat_128x128x16_2x2w_m32", 128, 128, 16, 2, 2, 8, 8, false, 1, 1, 32)     \
  X(7, "cat_128x128x32_2x2w_m16", 128, 128, 32, 2, 2, 16, 8, false, 1, 1, 16)    \
  X(8, "cat_256x128x16_4x2w_m32", 256, 128, 16, 4, 2, 8, 8, true, 1, 1, 32)      \
  X(9, "cat_128x256x16_2x4w_m16", 128, 256, 16, 2, 4, 8, 8, true, 1, 1, 16)

#define SGEMM_CATALOGUE_SIZE 10
