// Small-M kernel instances for 2 MFMA step(s) per group (g = 64), bfloat16.
#define W4A16_JPG 2
#define W4A16_BF 1
#include "w4a16_small_inst.inc"
