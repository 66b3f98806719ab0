// Small-M kernel instances for 4 MFMA step(s) per group (g >= 128), bfloat16.
#define W4A16_JPG 4
#define W4A16_BF 1
#include "w4a16_small_inst.inc"
