// fa_main_softcap.hip -- the soft-capped instantiations of the key-tile
// kernel of fa_main.hip (scores c * tanh(x / c), mha_bwd's softcap on the
// backward call-trace page), in a translation unit of their own so that they
// compile in parallel with the rest.
#define FA_MAIN_SOFTCAP_TU
#include "fa_main.hip"
