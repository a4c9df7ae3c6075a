// launch_table.hpp -- launch shape of the volume kernel per precision and
// polynomial order (LaunchCfg of volume_kernel.hpp), shared by the library's
// entry points and the measurement probes.
#pragma once

#include "volume_kernel.hpp"

namespace esdg {

// Launch shape per precision and order: EPB elements x NT threads per
// workgroup (the 3 (N+1)^2 line tasks of EPB elements fill whole waves as far
// as possible), whether the metric terms are staged in LDS, and whether the
// pair loop carries its series-only second form (volume term / with the
// surface term).  Chosen by timing on MI355X at the bubble, baroclinic and
// N=4 L=6 mesh sizes; the series form where it measured faster at the
// 4096- and 32,768-element sizes (it adds registers: at N <= 2 it gains
// nothing, and the fp64 N = 8 kernel would spill).
//
// At N = 3 and N = 7 (N+1 a power of two) the unpadded LDS node grid puts
// the lanes of a direction-1 or direction-2 line read on a few banks (up to
// 16 lanes per bank at N = 7); one pad value per row (N = 7) or three per
// plane (N = 3; fp32 with four per element and direction-major lines) spread
// them.  Waves whose lanes hold lines of two directions conflict too: at
// fp64 N = 6 and at N = 2 the 49 or 63 lines of each direction start on a
// 64-lane boundary (order 2), at the same 192 threads.  Other pads and orders were neutral
// to slower.  At fp64 N = 5 a 3-wave register cap on the volume kernel (168
// registers, a 36-byte spill) lets three workgroups share a CU instead of
// two; the kernel with the surface term at fp64 N = 3, 4 and 6 carries the
// series form under a 3-wave cap (no spill at N = 3, 108 and 28 bytes at
// N = 4 and 6; 2-10 % faster than the general form alone, while at N = 5 the
// same cap spills 244 bytes and runs 1.4x slower); at fp32 N = 4 and 5 a 5-wave cap on the kernel with the surface term
// (96 and 89 registers) does the same for five workgroups instead of four,
// and at fp32 N = 7 and 8 direction-3 lines that finish their nodes (25 and
// 32 KB of LDS) with 4-wave caps (128 registers) give five and four
// workgroups per CU instead of four and three.  At fp64 N = 4 and 5 and fp32
// N = 4 and 5 the general pair form forms its metric sums so that the
// compiler cannot hoist them above the form branch: at fp64 N = 4 the whole rhs's
// spill falls from 108 to 28 bytes, none left in the series form (1.4x on the
// rough baroclinic state, 1 % slower on the smooth bubble), and at fp64 N = 5
// the volume term's 36-byte spill goes (1.10x on the baroclinic state); the
// other orders measured neutral to slower with it.  With it the fp32 N = 4
// volume term fits 6 waves per SIMD (79 registers, no spill): six workgroups
// per CU, the 4096-element bubble in one round (1-2 % faster from 10,240
// elements up, unchanged on the bubble).  At fp32 N = 4 and 6 the staged
// value arrays start 64 slots apart (2.4 % and 12 % more LDS, occupancy
// unchanged), so a node's values come two per ds_read2st64_b32: half the LDS
// read instructions, 1.6-3.1 % faster; in fp64 the paired reads measured
// 2-5 % slower, and at fp32 N = 8 the change cost the fourth wave.
template <typename T, int N> struct Launch;
// LaunchCfg<EPB, NT, waves hint, metric staged in LDS, line cached in
// registers, line order (0 element-major, 1 direction-major, 2 direction-major
// with each direction on a 32-lane boundary), direction-3 lines finish the
// nodes, series form (volume term), series form (with the surface term), LDS
// pad per row, per plane, per element, waves hint with the surface term,
// lanes per line, distinct metric sums in the general form, value arrays
// 64 slots apart>
template <> struct Launch<double, 1> { using C = LaunchCfg<16, 192>; };                       // 192/192 lines
template <> struct Launch<double, 2> { using C = LaunchCfg<7, 192, 0, true, false, 2>; };     // 189/192
template <> struct Launch<double, 3> { using C = LaunchCfg<4, 192, 0, false, false, false, false, true, true, 0, 3, 0, 3>; };          // 192/192
template <> struct Launch<double, 4> { using C = LaunchCfg<3, 256, 0, false, false, true, false, true, true, 0, 0, 0, 3, 1, true>; };  // 225/256
template <> struct Launch<double, 5> { using C = LaunchCfg<2, 256, 3, false, false, true, false, true, true, 0, 0, 0, 0, 1, true>; };  // 216/256
template <> struct Launch<double, 6> { using C = LaunchCfg<1, 192, 0, true, false, 2, false, true, true, 0, 0, 0, 3>; };          // 147/192
template <> struct Launch<double, 7> { using C = LaunchCfg<1, 192, 0, false, false, true, true, true, true, 1>; };      // 192/192
template <> struct Launch<double, 8> { using C = LaunchCfg<1, 256, 0, false, false, true, true>; };                 // 243/256
template <> struct Launch<float, 1> { using C = LaunchCfg<16, 192>; };
template <> struct Launch<float, 2> { using C = LaunchCfg<7, 192, 0, true, false, 2>; };
template <> struct Launch<float, 3> { using C = LaunchCfg<4, 192, 0, true, false, 1, false, true, true, 0, 3, 4>; };
template <> struct Launch<float, 4> { using C = LaunchCfg<3, 256, 6, false, false, true, false, true, true, 0, 0, 0, 5, 1, true, true>; };
template <> struct Launch<float, 5> { using C = LaunchCfg<2, 256, 0, false, false, true, false, true, false, 0, 0, 0, 5, 1, true>; };
template <> struct Launch<float, 6> { using C = LaunchCfg<1, 192, 0, false, false, false, false, true, true, 0, 0, 0, 0, 1, false, true>; };
template <> struct Launch<float, 7> { using C = LaunchCfg<1, 192, 4, false, false, 1, true, true, true, 1, 0, 0, 4>; };
template <> struct Launch<float, 8> { using C = LaunchCfg<1, 256, 0, false, false, true, true, true, true, 0, 0, 0, 4>; };

}  // namespace esdg
