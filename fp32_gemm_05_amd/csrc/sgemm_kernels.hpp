// sgemm_kernels.hpp -- the HIP kernels of libsgemm for gfx950, one header per kernel family.
//
// kernel_common.hpp  shared pieces: argument block, workgroup -> tile map, slab loaders, MFMA step,
//                    epilogue, drain ordering, and the beta * C scale kernel;
// kernel_mfma.hpp    plain MFMA kernel (two LDS stages, register prefetch);
// kernel_pipe.hpp    the same with double-buffered LDS -> register fragments;
// kernel_deep.hpp    deep prefetch for about one workgroup per CU;
// kernel_splitk.hpp  in-workgroup split-K;
// kernel_direct.hpp  LDS-free kernel of small grids;
// kernel_dl.hpp      direct global -> LDS loads into a ring of LDS stages;
// kernel_valu.hpp    vector-FMA register microtile.
#pragma once

#include "kernel_common.hpp"
#include "kernel_mfma.hpp"
#include "kernel_pipe.hpp"
#include "kernel_deep.hpp"
#include "kernel_splitk.hpp"
#include "kernel_direct.hpp"
#include "kernel_dl.hpp"
#include "kernel_valu.hpp"
