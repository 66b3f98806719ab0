// Small-M kernel instances for 4 MFMA steps per group (g = 128 or 256).
#define W4A16_JPG 4
#include "w4a16_small_inst.inc"
