// The up projection's grouped GEMM, built from gemm_mfma.hip a second time with 64-deep
// k-tiles and loads staged through registers (namespace moe::kt64).
//
// Both operands of the up projection are K-contiguous (Xp rows and W1|W3 rows), and with
// 32-deep k-tiles each row of a k-tile is a 64-byte half cache line, so every line takes
// two L1-to-L2 requests.  64-deep k-tiles make each row one whole line; only two such
// stages fit in LDS, so the next-but-one k-tile waits in registers instead of a third
// stage.  Measured on the up projection at T = 32768, E = 256 (same results bit for bit):
// 14.98-15.10 ms -> 14.01-14.03 ms.  The other contractions (K-strided operands) were as
// fast or faster with the 32-deep direct-to-LDS loads, and keep them.
#define MOE_GEMM_KT64 1
#include "gemm_mfma.hip"
